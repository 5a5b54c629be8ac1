// pgq_kernels.hip -- gfx950 (CDNA4) kernels of libpgq: per-row symmetric quantization.
//
// Design (HBM-streaming, no dense contraction, so no MFMA):
//   * one 64-lane wavefront owns one row; a row of up to 2048 fp32 / 2048 bf16 values is
//     loaded once with 16-byte loads (global_load_dwordx4) and stays in VGPRs while its
//     clip is found, then every output is written once with coalesced stores;
//   * the clip is a wave-wide max (k = n), an iterated wave max for ranks near the top,
//     or an LDS-histogram radix select over the 31-bit magnitude patterns (8, 8, 8, 7
//     bits), exact for any k;
//   * persistent workgroups of 4 waves stride over tiles of rows, so a whole model (many
//     tensors of different widths) is one launch;
//   * longer rows stream through the same code in register-sized pieces, re-reading the
//     row (L2) for each select pass and for the output pass.
// Arithmetic follows the definition step by step in IEEE binary32 (correctly rounded
// divide, round-to-nearest-even, fp32 denormals kept), so the results are bit-exact:
//   x = w (* a_j), clip = k-th smallest |x|, s = fp16(clip / Q) (1 if 0),
//   code = clamp(rne(x / s), -Q, Q), dq = code * s (/ a_j),
//   STE mask = |x / s| <= Q + 1/2, grad_out = mask ? grad : +0,
//   SQWA mean = mean + (xhat - mean) / k.
// Sources: "Swiglu gating ... 10min/16MB Track" (PR #2159), Key Explored Modifications
// (per-row quantization, percentile clipping, fp16 passthrough, STE fake quantization);
// "SubSixteen v2" card (PR #69), sections Quantization and Other (6 bits, [-31, 31]);
// "12L ... Int6AWQ MixedBits" (PR #1495), Submission summary and Mixed-bit details;
// "Discriminative TTT + SLOT-24" card (PR #1414), Novel Contributions (SQWA).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pgq_desc.h"
#include "../../include/pgq.h"

namespace pgq {
namespace {

constexpr int kFastRank = 8;     // ranks up to this use the iterated wave max

#define GLB __attribute__((address_space(1)))

// Pointers taken from descriptors are generic; the data all live in global memory, so cast
// them once per row (uniform, scalar registers) and address lanes with 32-bit offsets.
template <class T>
__device__ __forceinline__ GLB T* gp(T* p) { return (GLB T*)p; }
template <class T>
__device__ __forceinline__ const GLB T* gp(const T* p) { return (const GLB T*)p; }

// Builtin vector types: 16-, 8-byte loads and stores through address-space-qualified pointers.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t fbits(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __uint_as_float(u); }

__device__ __forceinline__ uint16_t f2h(float f)
{
    _Float16 h = (_Float16)f;                  // v_cvt_f16_f32: round to nearest even, denormals kept
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ __forceinline__ uint16_t f2bf(float f)
{
    __bf16 b = (__bf16)f;                      // gfx950 v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, b);
}

// ---- wave-wide reductions with DPP (quad swaps, row mirrors, row broadcasts), result uniform --
// Every step pairs groups whose lanes already hold one value, so the same sequence serves max,
// sum and or.  Disabled rows read 0, the identity of all three.  Call with all 64 lanes active.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op)
{
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast15 -> rows 1, 3
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast31 -> rows 2, 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
struct OpMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };
struct OpSum { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpOr  { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a | b; } };
__device__ __forceinline__ uint32_t wave_max(uint32_t v) { return wave_reduce(v, OpMax()); }
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) { return wave_reduce(v, OpSum()); }
__device__ __forceinline__ uint32_t wave_or(uint32_t v) { return wave_reduce(v, OpOr()); }

__device__ __forceinline__ void lds_sync_wave()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// ---- element loads and stores --------------------------------------------------------------
// Addresses are a uniform (scalar) base plus a 32-bit byte offset per lane, so the hardware's
// scalar-base addressing applies (a row is shorter than 2^31 bytes).
template <class T>
__device__ __forceinline__ const GLB T* at(const GLB void* base, uint32_t byte_off)
{
    return reinterpret_cast<const GLB T*>(static_cast<const GLB uint8_t*>(base) + byte_off);
}
template <class T>
__device__ __forceinline__ GLB T* at(GLB void* base, uint32_t byte_off)
{
    return reinterpret_cast<GLB T*>(static_cast<GLB uint8_t*>(base) + byte_off);
}

// A row pointer advanced by a uniform number of elements of the input type.
template <int IN>
__device__ __forceinline__ const GLB void* offset_row(const GLB void* row, uint32_t elems)
{
    return static_cast<const GLB uint8_t*>(row) + (size_t)elems * (IN == IN_F32 ? 4 : 2);
}

// Streamed data (weights in, codes / dequant / means / gradients out) is touched once per
// launch: non-temporal loads and stores keep it from displacing other lines in L2.
template <class T>
__device__ __forceinline__ T ldnt(const GLB T* p) { return __builtin_nontemporal_load(p); }
template <class T>
__device__ __forceinline__ void stnt(GLB T* p, T v) { __builtin_nontemporal_store(v, p); }

// VEC consecutive elements starting at element e of a row
template <int IN, int VEC>
__device__ __forceinline__ void load_x(const GLB void* row, uint32_t e, float (&x)[VEC])
{
    if constexpr (IN == IN_F32) {
        if constexpr (VEC == 4) {
            const f32x4 v = ldnt(at<f32x4>(row, e * 4u));
            x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
        } else {
            static_assert(VEC == 1, "fp32 path uses VEC 4 or 1");
            x[0] = ldnt(at<float>(row, e * 4u));
        }
    } else {
        if constexpr (VEC == 8) {
            const u32x4 v = ldnt(at<u32x4>(row, e * 2u));
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) { x[2 * i] = bitsf(w[i] << 16); x[2 * i + 1] = bitsf(w[i] & 0xFFFF0000u); }
        } else {
            static_assert(VEC == 1, "bf16 path uses VEC 8 or 1");
            x[0] = bitsf((uint32_t)ldnt(at<uint16_t>(row, e * 2u)) << 16);
        }
    }
}

// int8 codes from integer-valued floats, at element e
template <int VEC>
__device__ __forceinline__ void store_codes(GLB int8_t* base, uint32_t e, const float (&r)[VEC])
{
    if constexpr (VEC == 1) {
        stnt(at<int8_t>(base, e), (int8_t)(int)r[0]);
    } else {
        uint32_t w[VEC / 4];
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i)
            w[i] = ((uint32_t)(int)r[4 * i] & 0xFFu) | (((uint32_t)(int)r[4 * i + 1] & 0xFFu) << 8) |
                   (((uint32_t)(int)r[4 * i + 2] & 0xFFu) << 16) | (((uint32_t)(int)r[4 * i + 3] & 0xFFu) << 24);
        if constexpr (VEC == 4) stnt(at<uint32_t>(base, e), w[0]);
        else stnt(at<u32x2>(base, e), u32x2{w[0], w[1]});
    }
}

// 6-bit code storage: four codes per three bytes, code 4g + t in bits 6t .. 6t+5 of the
// little-endian 24-bit group g (the export's int6 artifact layout).  Lane l holds the codes of
// chunk cu + l (cu uniform); VEC = 1 lanes pass their code to the first lane of their quad.
template <int VEC>
__device__ __forceinline__ void store_codes6(GLB uint8_t* row, uint32_t cu, int lane, const float (&r)[VEC],
                                             bool valid)
{
    auto field = [](float q) { return (uint32_t)(int)q & 0x3Fu; };
    auto put3 = [](GLB uint8_t* p, uint32_t w) {
        stnt(p, (uint8_t)(w & 0xFFu));
        stnt(p + 1, (uint8_t)((w >> 8) & 0xFFu));
        stnt(p + 2, (uint8_t)((w >> 16) & 0xFFu));
    };
    if constexpr (VEC == 1) {
        // every lane takes part (codes of lanes past the row are 0, the padding code)
        const uint32_t f = field(r[0]);
        const uint32_t f1 = (uint32_t)__shfl((int)f, lane + 1, 64);
        const uint32_t f2 = (uint32_t)__shfl((int)f, lane + 2, 64);
        const uint32_t f3 = (uint32_t)__shfl((int)f, lane + 3, 64);
        if (valid && (lane & 3) == 0) put3(row + 3u * ((cu + (uint32_t)lane) >> 2), f | (f1 << 6) | (f2 << 12) | (f3 << 18));
    } else {
        if (!valid) return;
#pragma unroll
        for (int g = 0; g < VEC / 4; ++g) {
            const uint32_t w = field(r[4 * g]) | (field(r[4 * g + 1]) << 6) | (field(r[4 * g + 2]) << 12) |
                               (field(r[4 * g + 3]) << 18);
            put3(row + 3u * ((cu + (uint32_t)lane) * (VEC / 4) + g), w);
        }
    }
}

template <int VEC>
__device__ __forceinline__ void store_f32(GLB float* base, uint32_t e, const float (&v)[VEC])
{
    if constexpr (VEC == 1) {
        stnt(at<float>(base, e * 4u), v[0]);
    } else {
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i)
            stnt(at<f32x4>(base, e * 4u + 16u * i), f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]});
    }
}

template <int VEC>
__device__ __forceinline__ void load_f32(const GLB float* base, uint32_t e, float (&v)[VEC])
{
    if constexpr (VEC == 1) {
        v[0] = ldnt(at<float>(base, e * 4u));
    } else {
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) {
            const f32x4 t = ldnt(at<f32x4>(base, e * 4u + 16u * i));
            v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
        }
    }
}

// 16-bit values (fp16 or bf16 bit patterns) packed two per dword, at element e
template <int VEC>
__device__ __forceinline__ void store_u16(GLB uint16_t* base, uint32_t e, const uint16_t (&h)[VEC])
{
    if constexpr (VEC == 1) {
        stnt(at<uint16_t>(base, e * 2u), h[0]);
    } else {
        uint32_t w[VEC / 2];
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i) w[i] = (uint32_t)h[2 * i] | ((uint32_t)h[2 * i + 1] << 16);
        if constexpr (VEC == 4) stnt(at<u32x2>(base, e * 2u), u32x2{w[0], w[1]});
        else stnt(at<u32x4>(base, e * 2u), u32x4{w[0], w[1], w[2], w[3]});
    }
}

template <int VEC>
__device__ __forceinline__ void load_u16(const GLB uint16_t* base, uint32_t e, uint16_t (&h)[VEC])
{
    if constexpr (VEC == 1) {
        h[0] = ldnt(at<uint16_t>(base, e * 2u));
    } else {
        static_assert(VEC == 8, "16-bit vector loads are 8 wide");
        const u32x4 v = ldnt(at<u32x4>(base, e * 2u));
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { h[2 * i] = (uint16_t)(w[i] & 0xFFFF); h[2 * i + 1] = (uint16_t)(w[i] >> 16); }
    }
}

// ---- the clip: the r-th largest magnitude key of the row (keys = |x| bit patterns) -------------
// `each(f)` calls f(key, valid) for every element slot this lane owns.
// One wave over a 256-bin digit histogram: the bin holding the rem-th largest key (bins count
// keys by digit, the largest digit last) and the number of keys in the bins above it.  All
// lanes active; results uniform.
// h: this lane's bins 4 lane .. 4 lane + 3.
__device__ __forceinline__ void radix_digit_bins(const uint32_t (&h)[4], uint32_t rem, int lane, uint32_t& digit,
                                                 uint32_t& above)
{
    const uint32_t s = h[0] + h[1] + h[2] + h[3];
    uint32_t inc = s;                       // sum over lanes >= lane
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = (uint32_t)__shfl_down((int)inc, off, 64);
        if (lane + off < 64) inc += v;
    }
    uint32_t run = inc - s;                 // count of keys in the bins above this lane's bins
    int found = -1;
    uint32_t abv = 0;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
        if (found < 0 && run < rem && run + h[b] >= rem) { found = 4 * lane + b; abv = run; }
        run += h[b];
    }
    const uint64_t bal = __ballot(found >= 0);
    const int src = bal ? __ffsll((unsigned long long)bal) - 1 : 0;
    digit = (uint32_t)__shfl(found, src, 64);
    above = (uint32_t)__shfl((int)abv, src, 64);
}

template <class HistPtr>
__device__ __forceinline__ void radix_digit(HistPtr hist, uint32_t rem, int lane, uint32_t& digit, uint32_t& above)
{
    uint32_t h[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) h[b] = hist[4 * lane + b];
    radix_digit_bins(h, rem, lane, digit, above);
}

// The k-th largest (1 <= k <= 64) of the 64 values the lanes hold: a lane whose value has fewer
// than k values above it and at least k at or above it holds the answer.  All lanes active.
__device__ __forceinline__ uint32_t rank_select64(uint32_t v, uint32_t k)
{
    uint32_t gt = 0, ge = 0;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
        const uint32_t u = (uint32_t)__builtin_amdgcn_readlane((int)v, j);
        gt += u > v ? 1u : 0u;
        ge += u >= v ? 1u : 0u;
    }
    const uint64_t hit = __ballot(gt < k && k <= ge);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, (int)__builtin_ctzll(hit));
}

template <class Each>
__device__ __forceinline__ uint32_t kth_largest(Each&& each, int64_t r, uint32_t* hist, int lane)
{
    if (r <= kFastRank) {
        // iterated maximum: strip the largest distinct magnitudes until r elements are covered.
        // One pass per round: the count of the current maximum m and the largest key below it.
        uint32_t m = 0;
        each([&](uint32_t k, bool ok) { if (ok) m = max(m, k); });
        m = wave_max(m);
        uint32_t rem = (uint32_t)r;
        // each round removes at least one element, so r rounds always suffice
        for (int round = 0; round < kFastRank && rem > 1; ++round) {
            uint32_t c = 0, below = 0;
            each([&](uint32_t k, bool ok) {
                c += (ok && k == m) ? 1u : 0u;
                if (ok && k < m) below = max(below, k);
            });
            c = wave_sum(c);
            if (c >= rem) return m;
            rem -= c;
            m = wave_max(below);
        }
        return m;
    }
    if (r <= 64) {
        // candidate select.  The r-th largest of the 64 lane maxima, t0, is a lower bound of the
        // answer (those r maxima are elements >= t0), so the answer is the r-th largest of the
        // elements >= t0.  When there are at most 64 of them (the usual case for r <= 64 unless
        // many keys tie), they are packed one per lane through LDS and ranked directly.
        uint32_t lm = 0;                       // a lane with no element offers 0 (<= every key)
        each([&](uint32_t k, bool ok) { if (ok) lm = max(lm, k); });
        const uint32_t t0 = rank_select64(lm, (uint32_t)r);
        uint32_t c = 0;
        each([&](uint32_t k, bool ok) { c += (ok && k >= t0) ? 1u : 0u; });
        c = wave_sum(c);
        if (c <= 64) {
            uint32_t base = 0;                 // uniform: candidates already packed
            each([&](uint32_t k, bool ok) {
                const bool cand = ok && k >= t0;
                const uint64_t b = __ballot(cand);
                const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
                if (cand) hist[base + below] = k;
                base += (uint32_t)__builtin_popcountll(b);
            });
            lds_sync_wave();
            const uint32_t v = (uint32_t)lane < c ? hist[lane] : 0u;   // padding ranks last
            lds_sync_wave();
            return rank_select64(v, (uint32_t)r);
        }
    }
    // radix select, most significant digit first: bits 30..23, 22..15, 14..7, 6..0, with a
    // 256-bin histogram per wave in LDS
    uint32_t prefix = 0, pmask = 0;
    uint32_t rem = (uint32_t)r;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = pass == 0 ? 23 : pass == 1 ? 15 : pass == 2 ? 7 : 0;
        for (int b = lane; b < 256; b += 64) hist[b] = 0;
        lds_sync_wave();
        each([&](uint32_t k, bool ok) {
            if (ok && (k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 0xFFu], 1u);
        });
        lds_sync_wave();
        uint32_t digit, above;
        radix_digit(hist, rem, lane, digit, above);
        lds_sync_wave();
        rem -= above;
        prefix |= digit << shift;
        pmask |= 0xFFu << shift;
    }
    return prefix & 0x7FFFFFFFu;
}

__device__ __forceinline__ float row_scale(float clip, int Q, uint16_t& s16, uint32_t& st)
{
    const float s32 = clip / (float)Q;         // correctly rounded binary32 divide
    uint16_t b = f2h(s32);
    if ((b & 0x7FFFu) == 0) b = 0x3C00u;       // scale 1 when fp16(clip / Q) is zero
    if ((b & 0x7FFFu) == 0x7C00u) st |= PGQ_DEV_SCALE_OVF;
    s16 = b;
    return h2f(b);
}

struct RowCtx {
    float sf;       // fp32 value of the fp16 scale
    float rinv;     // fl32(1 / sf)
    float Qf;       // Q
    float Qc;       // Q + 1: clamp for the reciprocal estimate
    float L;        // (Q + 1/2) * sf, exact: the STE mask is |x| <= L
    float kf;       // SQWA snapshot index
    int k;
    int fq_mode;
};

__device__ __forceinline__ void set_scale(RowCtx& rc, float sf)
{
    rc.sf = sf;
    rc.rinv = 1.0f / sf;                                  // correctly rounded
    rc.L = ((2.0f * rc.Qf + 1.0f) * sf) * 0.5f;           // (2Q+1) * s has <= 19 bits: exact
}

// code = clamp(rne(x / s), -Q, Q), bit-identical to rounding the correctly rounded quotient:
// y = x * fl32(1/s) is within 2^-15.9 of x / s whenever |x / s| <= Q + 2 (relative error
// <= 2^-23), so rint(y) is the nearest integer to x / s unless y lies within 2^-12 of a
// half-integer.  A fl32 quotient can only equal a half-integer h (|h| < 2^12) when x / s == h
// (s has 11 significant bits, x 24), so rne(fl32(x / s)) is the exact rounding of x / s.
// Chunks with any near-tie lane are recomputed with the correctly rounded divide itself.
// Codes are integers held in floats; zero is kept as +0 so that code * s is +0, as it is for
// an integer code converted back to binary32.
template <int VEC>
__device__ __forceinline__ void quant_chunk(const float (&x)[VEC], const RowCtx& rc, float (&r)[VEC])
{
    bool near = false;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        float y = x[v] * rc.rinv;
        y = __builtin_amdgcn_fmed3f(y, -rc.Qc, rc.Qc);
        const float q0 = __builtin_rintf(y);
        near |= fabsf(fabsf(y - q0) - 0.5f) < 0x1p-12f;
        r[v] = __builtin_amdgcn_fmed3f(q0, -rc.Qf, rc.Qf) + 0.0f;   // + 0 turns a -0 code into +0
    }
    if (__ballot(near)) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const float t = x[v] / rc.sf;
            r[v] = fminf(fmaxf(__builtin_rintf(t), -rc.Qf), rc.Qf) + 0.0f;
        }
    }
}

// Uniform per-row output pointers (global address space).
struct RowOut {
    GLB int8_t* codes;
    GLB uint8_t* packed;      // 6-bit code storage instead of codes
    GLB void* dq;
    GLB float* mean;
    GLB uint8_t* mask;
    const GLB uint16_t* grad;
    GLB uint16_t* gout;
    bool dq_f32;
};

__device__ __forceinline__ RowOut row_out(const Desc& d, int64_t row)
{
    const int64_t o = row * d.cols;
    RowOut ro;
    const bool pack6 = (d.flags & DF_PACK6) != 0;
    ro.codes = d.codes && !pack6 ? gp(d.codes) + o : nullptr;
    ro.packed = d.codes && pack6 ? (GLB uint8_t*)gp(d.codes) + row * (3 * ((d.cols + 3) >> 2)) : nullptr;
    ro.dq_f32 = d.dq_dtype == IN_F32;
    ro.dq = d.dq ? (ro.dq_f32 ? (GLB void*)(gp(static_cast<float*>(d.dq)) + o)
                              : (GLB void*)(gp(static_cast<uint16_t*>(d.dq)) + o))
                 : nullptr;
    ro.mean = d.mean ? gp(d.mean) + o : nullptr;
    ro.mask = d.mask ? gp(d.mask) + row * ((d.cols + 7) >> 3) : nullptr;
    ro.grad = d.grad ? gp(d.grad) + o : nullptr;
    ro.gout = d.grad_out ? gp(d.grad_out) + o : nullptr;
    return ro;
}

// Second input stream of a chunk, loaded together with the weights so that its latency is not
// paid again after the row's clip is known: the running mean (SQWA, k > 1) or the upstream
// gradient (STE forward + backward).
template <int MODE, int VEC>
struct Aux {
    float m[MODE == MODE_SQWA ? VEC : 1];
    uint16_t g[MODE == MODE_FQ ? VEC : 1];
};

template <int MODE, int VEC>
__device__ __forceinline__ void load_aux(const RowOut& ro, uint32_t cu, int lane, const RowCtx& rc, bool valid,
                                         Aux<MODE, VEC>& ax)
{
    if constexpr (MODE == MODE_SQWA) {
        if (rc.k > 1 && valid) load_f32<VEC>(ro.mean + cu * VEC, (uint32_t)lane * VEC, ax.m);
    } else if constexpr (MODE == MODE_FQ) {
        if (rc.fq_mode == PGQ_FQ_FWD_BWD && valid) load_u16<VEC>(ro.grad + cu * VEC, (uint32_t)lane * VEC, ax.g);
    }
}

// ---- outputs of one chunk: lane l owns VEC elements at (cu + l) * VEC of the row -------------
// cu is uniform: it moves the scalar base pointers, and every lane adds the same small offset
// lane * VEC, so all chunks of a row share one offset register.
template <int MODE, bool AWQ, int VEC>
__device__ __forceinline__ void chunk_out(const RowOut& ro, uint32_t cu, const float (&x)[VEC],
                                          const float (&a)[VEC], const float (&ainv)[VEC], bool has_awq,
                                          const RowCtx& rc, bool valid, int lane, const Aux<MODE, VEC>& ax)
{
    const uint32_t eu = cu * VEC;                 // uniform element offset of the chunk group
    const uint32_t e = (uint32_t)lane * VEC;      // lane's element offset within it
    float r[VEC];
    quant_chunk<VEC>(x, rc, r);
    float dq[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        dq[v] = r[v] * rc.sf;                     // exact (<= 8 + 11 significant bits); +0 for code 0
        if constexpr (AWQ) {
            // fl32(dq / a) from the correctly rounded reciprocal ainv = fl32(1/a): one product and
            // one remainder correction (Markstein).  Exact for every numerator of <= 18 and
            // denominator of <= 11 significant bits (no under/overflow is reachable here).
            if (has_awq) {
                const float q = dq[v] * ainv[v];
                const float rem = __builtin_fmaf(-q, a[v], dq[v]);
                dq[v] = __builtin_fmaf(rem, ainv[v], q);
            }
        }
    }
    if constexpr (is_export<MODE>) {
        if constexpr (MODE == MODE_EXPORT6) {
            if (ro.packed) store_codes6<VEC>(ro.packed, cu, lane, r, valid);
        }
        if (!valid) return;
        if (ro.codes) store_codes<VEC>(ro.codes + eu, e, r);
        if (ro.dq) {
            if (ro.dq_f32) {
                store_f32<VEC>(static_cast<GLB float*>(ro.dq) + eu, e, dq);
            } else {
                uint16_t h[VEC];
#pragma unroll
                for (int v = 0; v < VEC; ++v) h[v] = f2bf(dq[v]);
                store_u16<VEC>(static_cast<GLB uint16_t*>(ro.dq) + eu, e, h);
            }
        }
    } else if constexpr (MODE == MODE_SQWA) {
        if (!valid) return;
        GLB float* mp = ro.mean + eu;
        if (rc.k == 1) {
            store_f32<VEC>(mp, e, dq);
        } else {
            float m[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const float diff = dq[v] - ax.m[v];
                const float step = diff / rc.kf;
                m[v] = ax.m[v] + step;
            }
            store_f32<VEC>(mp, e, m);
        }
    } else if constexpr (MODE == MODE_FQ) {
        bool keep[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) keep[v] = fabsf(x[v]) <= rc.L;
        // mask bits: bit j % 8 of byte j / 8 of the row
        if (ro.mask) {
            if constexpr (VEC == 8) {
                if (valid) {
                    uint32_t byte = 0;
#pragma unroll
                    for (int v = 0; v < 8; ++v) byte |= keep[v] ? (1u << v) : 0u;
                    *at<uint8_t>(ro.mask + cu, (uint32_t)lane) = (uint8_t)byte;
                }
            } else {
                // element c = 64 * i + lane: the 64 lanes give 8 whole mask bytes
                const uint64_t bal = __ballot(valid && keep[0]);
                const uint32_t byte0 = cu >> 3;
                // lane b < 8 writes byte b of the group when that byte holds an element of the row
                const bool own = __shfl(valid ? 1 : 0, 8 * (lane & 7), 64) != 0;
                if (lane < 8 && own) *at<uint8_t>(ro.mask + byte0, (uint32_t)lane) = (uint8_t)(bal >> (8 * lane));
            }
        }
        if (!valid) return;
        uint16_t h[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) h[v] = f2bf(dq[v]);
        if (ro.dq) store_u16<VEC>(static_cast<GLB uint16_t*>(ro.dq) + eu, e, h);
        if (ro.codes) store_codes<VEC>(ro.codes + eu, e, r);
        if (rc.fq_mode == PGQ_FQ_FWD_BWD) {
            uint16_t g[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) g[v] = keep[v] ? ax.g[v] : (uint16_t)0;
            store_u16<VEC>(ro.gout + eu, e, g);
        }
    }
}

// AWQ multipliers of lane l's columns in chunk group cu (cu uniform)
template <int VEC>
__device__ __forceinline__ void load_awq(const GLB float* s_row, GLB uint16_t* a_out, uint32_t cu, int lane,
                                         float (&a)[VEC], float (&ainv)[VEC], uint32_t& st)
{
    float s[VEC];
    load_f32<VEC>(s_row + cu * VEC, (uint32_t)lane * VEC, s);
    uint16_t h[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        if (!(s[v] > 0.0f) || !(s[v] <= 3.402823466e38f)) st |= PGQ_DEV_BAD_AWQ;
        h[v] = f2h(__builtin_sqrtf(s[v]));       // correctly rounded sqrt, then fp16
        a[v] = h2f(h[v]);
        ainv[v] = 1.0f / a[v];                    // correctly rounded divide
    }
    if (a_out) store_u16<VEC>(a_out + cu * VEC, (uint32_t)lane * VEC, h);
}

// Multipliers of lane l's columns in chunk group cu from the workgroup's LDS table.  The table
// holds a_j in [0, kRegCols_F32) and fl32(1/a_j) in [kRegCols_F32, 2 kRegCols_F32), both padded
// with 1.0 past the row up to the register tile's extent, so no lane needs a bound.
template <int VEC>
__device__ __forceinline__ void lds_awq(const float* awq_lds, uint32_t cu, int lane, float (&a)[VEC])
{
    const uint32_t c = cu + (uint32_t)lane;
    if constexpr (VEC % 4 == 0) {
#pragma unroll
        for (int v = 0; v < VEC; v += 4) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(awq_lds + c * VEC + v);
            a[v] = t[0]; a[v + 1] = t[1]; a[v + 2] = t[2]; a[v + 3] = t[3];
        }
    } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) a[v] = awq_lds[c * VEC + v];
    }
}

// Extent of the AWQ table: the register tile's chunks cover cols rounded up to 64 * VEC, and
// VEC divides 8 and kRegCols_F32 is a multiple of 512.
__device__ __forceinline__ int awq_extent(int64_t cols)
{
    return (int)min((cols + 511) & ~(int64_t)511, (int64_t)kRegCols_F32);
}

// All threads of the workgroup: a_j = fp16(sqrt(s_j)) for the tensor's columns into LDS; the
// workgroup holding row 0 also writes the fp16 multipliers out.
__device__ __forceinline__ void fill_awq_lds(const Desc& d, bool write_out, float* awq_lds, uint32_t& st)
{
    const GLB float* s = gp(d.awq_s);
    GLB uint16_t* out = (write_out && d.awq_out) ? gp(d.awq_out) : nullptr;
    const int cols = (int)d.cols;
    const int ext = awq_extent(d.cols);
    for (int j = threadIdx.x; j < ext; j += kBlock) {
        float a = 1.0f, y = 1.0f;
        if (j < cols) {
            const float v = s[j];
            if (!(v > 0.0f) || !(v <= 3.402823466e38f)) st |= PGQ_DEV_BAD_AWQ;
            const uint16_t h = f2h(__builtin_sqrtf(v));      // correctly rounded sqrt, then fp16
            a = h2f(h);
            y = 1.0f / a;                                    // correctly rounded divide
            if (out) out[j] = h;
        }
        awq_lds[j] = a;
        awq_lds[kRegCols_F32 + j] = y;
    }
}

// ---- a group of R consecutive rows of one tensor (integer kinds) ------------------------------
// The register tile holds NCHT chunks per lane.  A row needing NCHT / R chunks or fewer is
// processed R rows at a time: every row's loads are issued before the first reduction, so a
// wave keeps R rows in flight.  Rows longer than the tile (R = 1 only) stream in pieces.
// EXACT: NCH is exactly ceil(chunks / 64) for this tensor, so chunks 0 .. NCH-2 are full and
// only the last needs a per-lane bound; otherwise NCH is the tile share and chunks are guarded.
// awq_lds: the tensor's AWQ multipliers a_j, computed once per workgroup into LDS (every
// tensor with AWQ whose rows fit the register tile); longer rows compute them per chunk.
template <int MODE, bool AWQ, bool SEL, bool LONG, int IN, int VEC, int R, int NCH, bool EXACT>
__device__ __forceinline__ void rows_quant(const Desc& d, int64_t row0, int nrows, int lane, uint32_t* hist,
                                           const float* awq_lds, const KArgs& ka, uint32_t& st)
{
    constexpr int NCHT = (VEC == 1) ? 16 : ((IN == IN_F32) ? 8 : 4);   // register tile, chunks per lane
    static_assert(NCH * R <= NCHT, "the group fits the register tile");
    static_assert(64 * NCHT * VEC == (VEC == 1 ? kRegCols_Scalar : (IN == IN_F32 ? kRegCols_F32 : kRegCols_BF16)),
                  "register tile must match the host's long-row threshold");
    const int nchunk = (int)(d.cols / VEC);
    const size_t esz = IN == IN_F32 ? 4 : 2;
    const bool has_awq = AWQ && d.awq_s != nullptr;
    const GLB float* s_row = has_awq ? gp(d.awq_s) : nullptr;
    GLB uint16_t* a_out = (has_awq && row0 == 0 && d.awq_out) ? gp(d.awq_out) : nullptr;

    RowCtx rc;
    rc.Qf = (float)d.Q;
    rc.Qc = (float)d.Q + 1.0f;
    rc.k = ka.sqwa_k;
    rc.kf = (float)ka.sqwa_k;
    rc.fq_mode = ka.fq_mode;

    if (R > 1 || !LONG || nchunk <= 64 * NCH) {
        static_assert(!EXACT || !LONG, "exact-width groups never stream");
        float x[R][NCH][VEC];
        Aux<MODE, VEC> ax[R][NCH];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r < nrows) {
                const RowOut ro = row_out(d, row0 + r);
#pragma unroll
                for (int i = 0; i < NCH; ++i)
                    if (EXACT || 64 * i < nchunk)
                        load_aux<MODE, VEC>(ro, 64u * i, lane, rc, (EXACT && i < NCH - 1) || lane + 64 * i < nchunk,
                                            ax[r][i]);
                const GLB void* wrow = (const GLB uint8_t*)gp(d.w) + (size_t)((row0 + r) * d.ld) * esz;
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    if (EXACT || 64 * i < nchunk) {
                        const uint32_t c = (uint32_t)(lane + 64 * i);
                        if ((EXACT && i < NCH - 1) || (int)c < nchunk) {
                            load_x<IN, VEC>(offset_row<IN>(wrow, 64u * i * VEC), (uint32_t)lane * VEC, x[r][i]);
                        } else {
#pragma unroll
                            for (int v = 0; v < VEC; ++v) x[r][i][v] = 0.0f;
                        }
                    }
                }
            }
        }
        if constexpr (AWQ) {
            if (has_awq) {
                // the column multipliers are the same for every row: read them from LDS
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    if (EXACT || 64 * i < nchunk) {
                        float a[VEC];
                        lds_awq<VEC>(awq_lds, 64u * i, lane, a);
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int v = 0; v < VEC; ++v) x[r][i][v] = x[r][i][v] * a[v];
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r < nrows) {
                const int64_t row = row0 + r;
                uint32_t ck;
                if (d.flags & DF_TENSOR) {
                    ck = gp(d.tstate)->key;         // the whole-tensor clip, selected beforehand
                } else {
                    uint32_t mx = 0;
#pragma unroll
                    for (int i = 0; i < NCH; ++i)
                        if (EXACT || 64 * i < nchunk)
#pragma unroll
                            for (int v = 0; v < VEC; ++v) mx = max(mx, fbits(x[r][i][v]) & 0x7FFFFFFFu);   // padding is +0
                    mx = wave_max(mx);
                    if (mx >= 0x7F800000u) st |= PGQ_DEV_NONFINITE;
                    ck = mx;
                    if constexpr (SEL) {
                        if (d.rank_top > 1) {
                            auto each = [&](auto&& f) {
#pragma unroll
                                for (int i = 0; i < NCH; ++i)
                                    if (EXACT || 64 * i < nchunk) {
                                        const bool ok = (EXACT && i < NCH - 1) || lane + 64 * i < nchunk;
#pragma unroll
                                        for (int v = 0; v < VEC; ++v) f(fbits(x[r][i][v]) & 0x7FFFFFFFu, ok);
                                    }
                            };
                            ck = kth_largest(each, d.rank_top, hist, lane);
                        }
                    }
                }
                uint16_t s16;
                set_scale(rc, row_scale(bitsf(ck), d.Q, s16, st));
                if (lane == 0 && d.scales && (row == 0 || !(d.flags & DF_TENSOR))) gp(d.scales)[row] = s16;
                const RowOut ro = row_out(d, row);
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    if (EXACT || 64 * i < nchunk) {
                        const uint32_t c = (uint32_t)(lane + 64 * i);
                        float ai[VEC], yi[VEC];
                        if constexpr (AWQ) {
                            if (has_awq) {
                                lds_awq<VEC>(awq_lds, 64u * i, lane, ai);
                                lds_awq<VEC>(awq_lds + kRegCols_F32, 64u * i, lane, yi);
                            }
                        }
                        const bool ok = (EXACT && i < NCH - 1) || (int)c < nchunk;
                        chunk_out<MODE, AWQ, VEC>(ro, 64u * i, x[r][i], ai, yi, has_awq, rc, ok, lane, ax[r][i]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
    } else if constexpr (LONG && R == 1) {
        // long row: stream it in pieces; every select pass and the output pass re-read it
        const int64_t row = row0;
        const GLB void* wrow = (const GLB uint8_t*)gp(d.w) + (size_t)(row * d.ld) * esz;
        const RowOut ro = row_out(d, row);
        // cu: uniform chunk base of the piece; lane l takes chunk cu + l
        auto load_chunk = [&](uint32_t cu, float (&x)[VEC], float (&a)[VEC], float (&ainv)[VEC],
                              GLB uint16_t* aw) {
            load_x<IN, VEC>(offset_row<IN>(wrow, cu * VEC), (uint32_t)lane * VEC, x);
            if (has_awq) {
                load_awq<VEC>(s_row, aw, cu, lane, a, ainv, st);
#pragma unroll
                for (int v = 0; v < VEC; ++v) x[v] = x[v] * a[v];
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v) { a[v] = 1.0f; ainv[v] = 1.0f; }
            }
        };
        uint32_t ck = 0;
        const bool tensor = (d.flags & DF_TENSOR) != 0;
        if (tensor) {
            ck = gp(d.tstate)->key;                 // the whole-tensor clip, selected beforehand
        } else {
            uint32_t mx = 0;
            for (int base = 0; base < nchunk; base += 64) {
                const uint32_t c = (uint32_t)(base + lane);
                if ((int)c < nchunk) {
                    float x[VEC], a[VEC], ainv[VEC];
                    load_chunk((uint32_t)base, x, a, ainv, a_out);
#pragma unroll
                    for (int v = 0; v < VEC; ++v) mx = max(mx, fbits(x[v]) & 0x7FFFFFFFu);
                }
            }
            mx = wave_max(mx);
            if (mx >= 0x7F800000u) st |= PGQ_DEV_NONFINITE;
            ck = mx;
        }
        if constexpr (SEL) {
            if (!tensor && d.rank_top > 1) {
                // f runs in uniform control flow (lanes past the row pass ok = false)
                auto each = [&](auto&& f) {
                    for (int base = 0; base < nchunk; base += 64) {
                        const bool ok = base + lane < nchunk;
                        float x[VEC], a[VEC], ainv[VEC];
                        if (ok) {
                            load_chunk((uint32_t)base, x, a, ainv, nullptr);
                        } else {
#pragma unroll
                            for (int v = 0; v < VEC; ++v) x[v] = 0.0f;
                        }
#pragma unroll
                        for (int v = 0; v < VEC; ++v) f(fbits(x[v]) & 0x7FFFFFFFu, ok);
                    }
                };
                ck = kth_largest(each, d.rank_top, hist, lane);
            }
        }
        uint16_t s16;
        set_scale(rc, row_scale(bitsf(ck), d.Q, s16, st));
        if (lane == 0 && d.scales && (row == 0 || !tensor)) gp(d.scales)[row] = s16;
        for (int base = 0; base < nchunk; base += 64) {
            const uint32_t c = (uint32_t)(base + lane);
            const bool ok = (int)c < nchunk;
            float x[VEC], a[VEC], ainv[VEC];
            if (ok) {
                load_chunk((uint32_t)base, x, a, ainv, nullptr);
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v) { x[v] = 0.0f; a[v] = 1.0f; ainv[v] = 1.0f; }
            }
            Aux<MODE, VEC> ax;
            load_aux<MODE, VEC>(ro, (uint32_t)base, lane, rc, ok, ax);
            chunk_out<MODE, AWQ, VEC>(ro, (uint32_t)base, x, a, ainv, has_awq, rc, ok, lane, ax);
        }
    }
}

// Run rows_quant with the group shape the host chose for this tensor.  Vector paths use the
// exact chunk count (d.nch) and group size (d.rgroup); the element-wise path splits the tile.
template <int MODE, bool AWQ, bool SEL, bool LONG, int IN, int VEC, int R, int NCH>
__device__ __forceinline__ void rows_exact(const Desc& d, int64_t row0, int nrows, int lane, uint32_t* hist,
                                           const float* awq_lds, const KArgs& ka, uint32_t& st)
{
    rows_quant<MODE, AWQ, SEL, false, IN, VEC, R, NCH, true>(d, row0, nrows, lane, hist, awq_lds, ka, st);
}

template <int MODE, bool AWQ, bool SEL, bool LONG, int IN, int VEC>
__device__ __forceinline__ void rows_quant_r(const Desc& d, int64_t row0, int nrows, int lane, uint32_t* hist,
                                             const float* awq_lds, const KArgs& ka, uint32_t& st)
{
    constexpr int NCHT = (VEC == 1) ? 16 : ((IN == IN_F32) ? 8 : 4);
    if constexpr (VEC == 1) {
        switch (d.rgroup) {
        case 8: rows_quant<MODE, AWQ, SEL, false, IN, VEC, 8, NCHT / 8, false>(d, row0, nrows, lane, hist, awq_lds, ka, st); break;
        case 4: rows_quant<MODE, AWQ, SEL, false, IN, VEC, 4, NCHT / 4, false>(d, row0, nrows, lane, hist, awq_lds, ka, st); break;
        case 2: rows_quant<MODE, AWQ, SEL, false, IN, VEC, 2, NCHT / 2, false>(d, row0, nrows, lane, hist, awq_lds, ka, st); break;
        default:
            for (int r = 0; r < nrows; ++r)
                rows_quant<MODE, AWQ, SEL, LONG, IN, VEC, 1, NCHT, false>(d, row0 + r, 1, lane, hist, awq_lds, ka, st);
            break;
        }
        return;
    } else {
        // (rgroup, nch) pairs the host produces: rgroup = NCHT / pow2ceil(nch), or 1
        const int key = d.rgroup * 16 + d.nch;
        if (d.nch == 0) {            // longer than the register tile: stream row by row
            if constexpr (LONG) {
                for (int r = 0; r < nrows; ++r)
                    rows_quant<MODE, AWQ, SEL, LONG, IN, VEC, 1, NCHT, false>(d, row0 + r, 1, lane, hist, awq_lds, ka, st);
            }
            return;
        }
        if constexpr (NCHT == 8) {
            switch (key) {
            case 8 * 16 + 1: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 8, 1>(d, row0, nrows, lane, hist, awq_lds, ka, st); return;
            case 4 * 16 + 2: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 4, 2>(d, row0, nrows, lane, hist, awq_lds, ka, st); return;
            case 2 * 16 + 3: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 2, 3>(d, row0, nrows, lane, hist, awq_lds, ka, st); return;
            case 2 * 16 + 4: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 2, 4>(d, row0, nrows, lane, hist, awq_lds, ka, st); return;
            default: break;
            }
        } else {
            switch (key) {
            case 4 * 16 + 1: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 4, 1>(d, row0, nrows, lane, hist, awq_lds, ka, st); return;
            case 2 * 16 + 2: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 2, 2>(d, row0, nrows, lane, hist, awq_lds, ka, st); return;
            default: break;
            }
        }
        // one row at a time with its exact chunk count
        for (int r = 0; r < nrows; ++r) {
            const int64_t row = row0 + r;
            switch (d.nch) {
            case 1: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 1, 1>(d, row, 1, lane, hist, awq_lds, ka, st); break;
            case 2: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 1, 2>(d, row, 1, lane, hist, awq_lds, ka, st); break;
            case 3: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 1, 3>(d, row, 1, lane, hist, awq_lds, ka, st); break;
            case 4: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 1, 4>(d, row, 1, lane, hist, awq_lds, ka, st); break;
            default:
                if constexpr (NCHT == 8) {
                    switch (d.nch) {
                    case 5: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 1, 5>(d, row, 1, lane, hist, awq_lds, ka, st); break;
                    case 6: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 1, 6>(d, row, 1, lane, hist, awq_lds, ka, st); break;
                    case 7: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 1, 7>(d, row, 1, lane, hist, awq_lds, ka, st); break;
                    default: rows_exact<MODE, AWQ, SEL, LONG, IN, VEC, 1, 8>(d, row, 1, lane, hist, awq_lds, ka, st); break;
                    }
                }
                break;
            }
        }
    }
}

// ---- fp16 passthrough row (export: fp16 out + optional fp32 decode; SQWA: fp16 round trip) ---
template <int MODE, int IN, int VEC>
__device__ __forceinline__ void row_passthrough(const Desc& d, int64_t row, int lane, const KArgs& ka, uint32_t& st)
{
    const int nchunk = (int)(d.cols / VEC);
    const size_t esz = IN == IN_F32 ? 4 : 2;
    const GLB void* wrow = (const GLB uint8_t*)gp(d.w) + (size_t)(row * d.ld) * esz;
    const int64_t o = row * d.cols;
    GLB uint16_t* hrow = d.f16_out ? gp(d.f16_out) + o : nullptr;
    GLB float* dqrow = d.dq ? gp(static_cast<float*>(d.dq)) + o : nullptr;
    GLB float* mrow = d.mean ? gp(d.mean) + o : nullptr;
    const float kf = (float)ka.sqwa_k;
    for (int base = 0; base < nchunk; base += 64) {
        const uint32_t c = (uint32_t)(base + lane);
        if ((int)c >= nchunk) break;
        const uint32_t e = c * VEC;
        float x[VEC];
        load_x<IN, VEC>(wrow, e, x);
        uint16_t h[VEC];
        float y[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            h[v] = f2h(x[v]);
            y[v] = h2f(h[v]);
            if (!(fabsf(x[v]) <= 3.402823466e38f)) st |= PGQ_DEV_NONFINITE;
            else if ((h[v] & 0x7FFFu) == 0x7C00u) st |= PGQ_DEV_F16_OVF;
        }
        if constexpr (is_export<MODE>) {
            if (hrow) store_u16<VEC>(hrow, e, h);
            if (dqrow) store_f32<VEC>(dqrow, e, y);
        } else {
            if (ka.sqwa_k == 1) {
                store_f32<VEC>(mrow, e, y);
            } else {
                float m[VEC];
                load_f32<VEC>(mrow, e, m);
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    const float diff = y[v] - m[v];
                    const float step = diff / kf;
                    m[v] = m[v] + step;
                }
                store_f32<VEC>(mrow, e, m);
            }
        }
    }
}

// ---- STE backward only: grad_out = mask ? grad : +0 --------------------------------------------
template <int VEC>
__device__ __forceinline__ void row_fq_bwd(const Desc& d, int64_t row, int lane)
{
    const int nchunk = (int)(d.cols / VEC);
    const RowOut ro = row_out(d, row);
    for (int base = 0; base < nchunk; base += 64) {
        const uint32_t c = (uint32_t)(base + lane);
        if ((int)c >= nchunk) break;
        const uint32_t e = c * VEC;
        uint16_t g[VEC];
        load_u16<VEC>(ro.grad, e, g);
        if constexpr (VEC == 8) {
            const uint32_t byte = ro.mask[c];
#pragma unroll
            for (int v = 0; v < 8; ++v) g[v] = ((byte >> v) & 1u) ? g[v] : (uint16_t)0;
        } else {
            const uint32_t byte = ro.mask[c >> 3];
            g[0] = ((byte >> (c & 7u)) & 1u) ? g[0] : (uint16_t)0;
        }
        store_u16<VEC>(ro.gout, e, g);
    }
}

// ---- weight averaging rows: fp32 state rows x cols, dense --------------------------------------
// EMA (Weight Averaging sections of the PR #1414 / PR #1202 cards, decay 0.997):
// e = fl32(fl32(d * e) + fl32(c * w)) with c = fl32(1 - d), or e = w on the first update.
// SWA (PR #69 card, 16 checkpoints): the running mean of the checkpoints, mean = w for k = 1,
// else fl32(mean + fl32(fl32(w - mean) / k)).  Pure streaming: U chunks per lane in flight.
template <int MODE, int IN, int VEC>
__device__ __forceinline__ void row_average(const Desc& d, int64_t row, int lane, const KArgs& ka, uint32_t& st)
{
    constexpr int U = VEC >= 8 ? 1 : VEC == 4 ? 2 : 8;
    const int nchunk = (int)(d.cols / VEC);
    const size_t esz = IN == IN_F32 ? 4 : 2;
    const GLB void* wrow = (const GLB uint8_t*)gp(d.w) + (size_t)(row * d.ld) * esz;
    GLB float* mrow = gp(d.mean) + row * d.cols;
    const bool copy = MODE == MODE_EMA ? ka.avg_init != 0 : ka.sqwa_k == 1;
    const float kf = (float)ka.sqwa_k;
    const uint32_t e = (uint32_t)lane * VEC;
    for (int base = 0; base < nchunk; base += 64 * U) {
        float x[U][VEC], m[U][VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cb = base + 64 * u;                 // uniform chunk base
            if (cb + lane < nchunk) {
                load_x<IN, VEC>(offset_row<IN>(wrow, (uint32_t)(cb * VEC)), e, x[u]);
                if (!copy) load_f32<VEC>(mrow + cb * VEC, e, m[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cb = base + 64 * u;
            if (cb + lane < nchunk) {
                float r[VEC];
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    if (copy) {
                        r[v] = x[u][v];
                    } else if constexpr (MODE == MODE_EMA) {
                        const float kept = ka.avg_d * m[u][v];
                        const float added = ka.avg_c * x[u][v];
                        r[v] = kept + added;
                    } else {
                        const float diff = x[u][v] - m[u][v];
                        const float step = diff / kf;
                        r[v] = m[u][v] + step;
                    }
                    if (!(fabsf(x[u][v]) <= 3.402823466e38f) || !(fabsf(r[v]) <= 3.402823466e38f))
                        st |= PGQ_DEV_NONFINITE;
                }
                store_f32<VEC>(mrow + cb * VEC, e, r);
            }
        }
    }
}

// ---- decode of one stored row (grouped whole-model decode) ---------------------------------------
// Integer kinds: x = code * s (/ a_j), the export's own dequant; fp16 passthrough: fp32 of the
// stored half.  Codes are int8 or 6-bit packed (DF_PACK6); lane l takes groups of four columns.
__device__ __forceinline__ void row_decode(const Desc& d, int64_t row, int lane)
{
    const int64_t cols = d.cols;
    const int64_t ngroups = (cols + 3) >> 2;
    GLB float* orow = gp(static_cast<float*>(d.dq)) + row * cols;
    if (d.kind == KIND_F16) {
        const GLB uint16_t* hrow = gp(d.f16_out) + row * cols;
        for (int64_t j = lane; j < cols; j += 64) stnt(orow + j, h2f(hrow[j]));
        return;
    }
    const bool packed = (d.flags & DF_PACK6) != 0;
    const bool vec = (d.flags & DF_VEC) != 0;
    const float s = h2f(gp(d.scales)[(d.flags & DF_TENSOR) ? 0 : row]);
    const GLB uint8_t* crow = (const GLB uint8_t*)gp(d.codes) + row * (packed ? 3 * ngroups : cols);
    const GLB uint16_t* awq = d.awq_out ? gp(d.awq_out) : nullptr;
    for (int64_t g = lane; g < ngroups; g += 64) {
        int32_t q[4];
        if (packed) {
            const uint32_t w = (uint32_t)crow[3 * g] | ((uint32_t)crow[3 * g + 1] << 8) | ((uint32_t)crow[3 * g + 2] << 16);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int32_t f = (int32_t)((w >> (6 * t)) & 0x3Fu);
                q[t] = f >= 32 ? f - 64 : f;
            }
        } else if (vec) {                                   // four int8 codes, 4-byte aligned
            const uint32_t w = *at<uint32_t>(crow, (uint32_t)(4 * g));
#pragma unroll
            for (int t = 0; t < 4; ++t) q[t] = (int32_t)(int8_t)((w >> (8 * t)) & 0xFFu);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) q[t] = 4 * g + t < cols ? (int32_t)(int8_t)crow[4 * g + t] : 0;
        }
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int64_t j = 4 * g + t;
            v[t] = (float)q[t] * s;
            if (awq && j < cols) v[t] = v[t] / h2f(awq[j]);    // correctly rounded divide
        }
        if (vec) {                                          // cols % 4 == 0, 16-byte aligned rows
            stnt(at<f32x4>(orow, (uint32_t)(16 * g)), f32x4{v[0], v[1], v[2], v[3]});
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (4 * g + t < cols) stnt(orow + 4 * g + t, v[t]);
        }
    }
}

template <int MODE, uint32_t F>
__device__ __forceinline__ void dispatch_rows(const Desc& d, int64_t row, int nrows, int lane, uint32_t* hist,
                                              const float* awq_lds, const KArgs& ka, uint32_t& st)
{
    constexpr bool AWQ = (F & F_AWQ) != 0;
    constexpr bool SEL = (F & F_SEL) != 0;
    constexpr bool LONG = (F & F_LONG) != 0;
    constexpr bool SCALAR = (F & F_SCALAR) != 0;
    const bool vec = (d.flags & DF_VEC) != 0;
    if constexpr (MODE == MODE_DECODE) {
        for (int r = 0; r < nrows; ++r) row_decode(d, row + r, lane);
    } else if constexpr (MODE == MODE_EMA || MODE == MODE_SWA) {
        for (int r = 0; r < nrows; ++r) {
            if constexpr ((F & F_F32) != 0) {
                if (d.in_dtype == IN_F32) {
                    if constexpr (SCALAR) {
                        if (!vec) { row_average<MODE, IN_F32, 1>(d, row + r, lane, ka, st); continue; }
                    }
                    row_average<MODE, IN_F32, 4>(d, row + r, lane, ka, st);
                    continue;
                }
            }
            if constexpr ((F & F_BF16) != 0) {
                if constexpr (SCALAR) {
                    if (!vec) { row_average<MODE, IN_BF16, 1>(d, row + r, lane, ka, st); continue; }
                }
                row_average<MODE, IN_BF16, 8>(d, row + r, lane, ka, st);
            }
        }
    } else if constexpr (MODE == MODE_FQ_BWD) {
        for (int r = 0; r < nrows; ++r) {
            if (vec) row_fq_bwd<8>(d, row + r, lane);
            else row_fq_bwd<1>(d, row + r, lane);
        }
    } else if constexpr (MODE == MODE_FQ) {
        if constexpr (SCALAR) {
            if (!vec) { rows_quant_r<MODE_FQ, false, SEL, LONG, IN_BF16, 1>(d, row, nrows, lane, hist, awq_lds, ka, st); return; }
        }
        rows_quant_r<MODE_FQ, false, SEL, LONG, IN_BF16, 8>(d, row, nrows, lane, hist, awq_lds, ka, st);
    } else {
        if constexpr ((F & F_PASS) != 0) {
            if (d.kind == KIND_F16) {
                if constexpr ((F & F_F32) != 0) {
                    if (d.in_dtype == IN_F32) {
                        for (int r = 0; r < nrows; ++r) {
                            if constexpr (SCALAR) {
                                if (!vec) { row_passthrough<MODE, IN_F32, 1>(d, row + r, lane, ka, st); continue; }
                            }
                            row_passthrough<MODE, IN_F32, 4>(d, row + r, lane, ka, st);
                        }
                        return;
                    }
                }
                if constexpr ((F & F_BF16) != 0) {
                    for (int r = 0; r < nrows; ++r) {
                        if constexpr (SCALAR) {
                            if (!vec) { row_passthrough<MODE, IN_BF16, 1>(d, row + r, lane, ka, st); continue; }
                        }
                        row_passthrough<MODE, IN_BF16, 8>(d, row + r, lane, ka, st);
                    }
                }
                return;
            }
        }
        if constexpr ((F & F_F32) != 0) {
            if (d.in_dtype == IN_F32) {
                if constexpr (SCALAR) {
                    if (!vec) { rows_quant_r<MODE, AWQ, SEL, LONG, IN_F32, 1>(d, row, nrows, lane, hist, awq_lds, ka, st); return; }
                }
                rows_quant_r<MODE, AWQ, SEL, LONG, IN_F32, 4>(d, row, nrows, lane, hist, awq_lds, ka, st);
                return;
            }
        }
        if constexpr ((F & F_BF16) != 0) {
            if constexpr (SCALAR) {
                if (!vec) { rows_quant_r<MODE, AWQ, SEL, LONG, IN_BF16, 1>(d, row, nrows, lane, hist, awq_lds, ka, st); return; }
            }
            rows_quant_r<MODE, AWQ, SEL, LONG, IN_BF16, 8>(d, row, nrows, lane, hist, awq_lds, ka, st);
        }
    }
}

// ---- whole-tensor clip select (per-tensor scales) ---------------------------------------------
// The clip of a DF_TENSOR tensor is the rank_top-th largest |x| over all its elements
// ("per-row / per-tensor quantization" with percentile clipping, PR #2159 Key Explored
// Modifications), found by a radix select over the key bits 30..23, 22..15, 14..7, 6..0, one
// launch per digit: every workgroup histograms the digits of its keys that match the digits
// chosen so far in LDS and adds the histogram into hist[pass] with device atomics.  The chosen
// digits are re-derived from the earlier passes' histograms at the start of each pass (the
// launch boundary makes them complete), so no workgroup waits on another and none needs a
// device-scope fence (on this chip that writes back and invalidates the XCD's L2).
// pgq_tensor_pick_kernel finishes.  rank_top = 1 is a single max pass.

// Digits 0 .. npass-1 of the select from a TState's histograms: the key prefix, its mask and
// the rank still to find among the keys that match it.  One wave, all lanes; uniform results.
__device__ __forceinline__ void tensor_prefix(const GLB TState* S, uint32_t rank, int npass, int lane,
                                              uint32_t& prefix, uint32_t& pmask, uint32_t& rem)
{
    prefix = 0;
    pmask = 0;
    rem = rank;
    uint32_t h[4][4];                               // every histogram's bins in one load round
#pragma unroll
    for (int p = 0; p < 4; ++p)
        if (p < npass) {
#pragma unroll
            for (int b = 0; b < 4; ++b) h[p][b] = S->hist[p][4 * lane + b];
        }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        if (p < npass) {
            const int shift = p == 0 ? 23 : p == 1 ? 15 : p == 2 ? 7 : 0;
            uint32_t digit, above;
            radix_digit_bins(h[p], rem, lane, digit, above);
            rem -= above;
            prefix |= digit << shift;
            pmask |= 0xFFu << shift;
        }
    }
}

// One pass over rows [row0, row0 + nrows) of the tensor.  Whole workgroup; wg_hist: kWaves x 256
// words of LDS.
template <int IN, int VEC>
__device__ __forceinline__ void tile_tensor_select(const Desc& d, int64_t row0, int64_t nrows, int wave, int lane,
                                                   uint32_t* wg_hist, const KArgs& ka, uint32_t& st)
{
    TState* S = d.tstate;
    const int pass = ka.tsel_pass;
    const bool absmax = d.rank_top == 1;
    if (absmax && pass > 0) return;                  // uniform: nothing left to select
    const int shift = pass == 0 ? 23 : pass == 1 ? 15 : pass == 2 ? 7 : 0;
    uint32_t prefix, pmask, rem;
    tensor_prefix(gp(S), (uint32_t)d.rank_top, absmax ? 0 : pass, lane, prefix, pmask, rem);
    const int tid = (int)threadIdx.x;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) wg_hist[256 * w + tid] = 0;   // one histogram per wave
    __syncthreads();
    uint32_t* my_hist = wg_hist + 256 * wave;       // waves do not contend for bins
    const int nchunk = (int)(d.cols / VEC);
    const size_t esz = IN == IN_F32 ? 4 : 2;
    const int64_t rend = min(row0 + nrows, d.rows);
    uint32_t m = 0, bad = 0;
    for (int64_t row = row0 + wave; row < rend; row += kWaves) {
        const GLB void* wrow = (const GLB uint8_t*)gp(d.w) + (size_t)(row * d.ld) * esz;
        for (int base = 0; base < nchunk; base += 64) {
            const int c = base + lane;
            if (c < nchunk) {
                float x[VEC];
                load_x<IN, VEC>(wrow, (uint32_t)c * VEC, x);
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    const uint32_t k = fbits(x[v]) & 0x7FFFFFFFu;
                    bad |= k >= 0x7F800000u ? 1u : 0u;
                    if (absmax) m = max(m, k);
                    else if ((k & pmask) == prefix) atomicAdd(&my_hist[(k >> shift) & 0xFFu], 1u);
                }
            }
        }
    }
    if (pass == 0 && bad) st |= PGQ_DEV_NONFINITE;
    if (absmax) {
        m = wave_max(m);
        if (lane == 0) wg_hist[wave] = m;           // absmax builds no histogram
    }
    __syncthreads();
    if (absmax) {
        if (tid == 0) atomicMax(&S->kmax, max(max(wg_hist[0], wg_hist[1]), max(wg_hist[2], wg_hist[3])));
    } else {
        const uint32_t c = wg_hist[tid] + wg_hist[256 + tid] + wg_hist[512 + tid] + wg_hist[768 + tid];
        if (c) atomicAdd(&S->hist[pass][tid], c);
    }
}

// A tile is tile_rows consecutive rows of one tensor; wave w takes groups of rgroup rows,
// groups interleaved over the four waves.
template <int MODE, uint32_t F>
__device__ __forceinline__ void do_tile(const Desc& d, int64_t row0, int wave, int lane, uint32_t* hist,
                                        float* awq_lds, const KArgs& ka, uint32_t& st)
{
    if constexpr (MODE == MODE_TSEL) {
        uint32_t* wg_hist = hist - 256 * wave;      // the workgroup's LDS histograms, 4 x 256 words
        const int64_t nrows = (int64_t)d.tile_rows * ka.tsel_group;   // row0 counts select tiles
        const bool vec = (d.flags & DF_VEC) != 0;
        if constexpr ((F & F_F32) != 0) {
            if (d.in_dtype == IN_F32) {
                if constexpr ((F & F_SCALAR) != 0) {
                    if (!vec) { tile_tensor_select<IN_F32, 1>(d, row0, nrows, wave, lane, wg_hist, ka, st); return; }
                }
                tile_tensor_select<IN_F32, 4>(d, row0, nrows, wave, lane, wg_hist, ka, st);
                return;
            }
        }
        if constexpr ((F & F_BF16) != 0) {
            if constexpr ((F & F_SCALAR) != 0) {
                if (!vec) { tile_tensor_select<IN_BF16, 1>(d, row0, nrows, wave, lane, wg_hist, ka, st); return; }
            }
            tile_tensor_select<IN_BF16, 8>(d, row0, nrows, wave, lane, wg_hist, ka, st);
        }
        return;
    }
    // AWQ multipliers for the whole tile, once (rows that fit the register tile read them from
    // LDS).  The condition is uniform over the workgroup, so every wave reaches the barriers.
    const float* lds = nullptr;
    if constexpr ((F & F_AWQ) != 0) {
        if (d.awq_s && d.kind != KIND_F16 && d.nch > 0) {
            __syncthreads();                    // readers of the previous tile's table are done
            fill_awq_lds(d, row0 == 0, awq_lds, st);
            __syncthreads();
            lds = awq_lds;
        } else if (d.awq_s && d.kind != KIND_F16 && d.rgroup > 0 && (d.flags & DF_VEC) == 0 &&
                   d.cols <= kRegCols_Scalar) {
            __syncthreads();
            fill_awq_lds(d, row0 == 0, awq_lds, st);
            __syncthreads();
            lds = awq_lds;
        }
    }
    const int R = d.rgroup;
    const int groups = d.tile_rows / (kWaves * R);
    for (int g = 0; g < groups; ++g) {
        const int64_t first = row0 + ((int64_t)g * kWaves + wave) * R;
        if (first < d.rows) {
            const int nrows = (int)min((int64_t)R, d.rows - first);
            dispatch_rows<MODE, F>(d, first, nrows, lane, hist, lds, ka, st);
        }
    }
}

// Copy the descriptor fields a mode uses into scalar registers in one round of scalar loads.
// Scalar loads return out of order, so each use waits for every outstanding one; loading all
// fields before the first branch (the empty asm consumes them) avoids a chain of dependent
// load rounds before the first row load.
template <int MODE, uint32_t F>
__device__ __forceinline__ Desc fetch_desc(const Desc* __restrict__ p)
{
    Desc d = *p;
    asm volatile("" ::"s"(d.rows), "s"(d.cols), "s"(d.ld), "s"(d.kind), "s"(d.flags), "s"(d.rgroup),
                 "s"(d.tile_rows), "s"(d.nch), "s"(d.w), "s"(d.Q));
    if constexpr (is_export<MODE>) asm volatile("" ::"s"(d.codes), "s"(d.scales), "s"(d.dq), "s"(d.dq_dtype));
    if constexpr (MODE == MODE_SQWA || MODE == MODE_EMA || MODE == MODE_SWA) asm volatile("" ::"s"(d.mean));
    if constexpr (MODE == MODE_TSEL) asm volatile("" ::"s"(d.tstate), "s"(d.rank_top), "s"(d.in_dtype));
    if constexpr (MODE == MODE_DECODE) asm volatile("" ::"s"(d.codes), "s"(d.scales), "s"(d.dq), "s"(d.f16_out), "s"(d.awq_out));
    if constexpr (is_export<MODE>) asm volatile("" ::"s"(d.tstate));
    if constexpr (MODE == MODE_FQ || MODE == MODE_FQ_BWD)
        asm volatile("" ::"s"(d.dq), "s"(d.scales), "s"(d.mask), "s"(d.grad), "s"(d.grad_out));
    if constexpr ((F & F_PASS) != 0 && is_export<MODE>) asm volatile("" ::"s"(d.f16_out));
    if constexpr ((F & F_SEL) != 0) asm volatile("" ::"s"(d.rank_top));
    if constexpr ((F & F_AWQ) != 0) asm volatile("" ::"s"(d.awq_s), "s"(d.awq_out));
    return d;
}

// Grouped launches: descriptors come from the table in the workspace through restrict-qualified
// pointers (read-only for the whole launch, so scalar loads).  F is the feature set compiled in.
// Occupancy floor for the lean streaming variants, chosen so the register budget still needs
// no scratch: 7 waves per SIMD (<= 72 VGPRs) for export rows, 5 (<= 96) for fp32 SQWA rows,
// which also keep a running mean in flight.  Measured: ~1% faster each; a floor that forces
// spilling (export at 8 waves, STE at 6) is slower.
template <int MODE, uint32_t F>
constexpr int kMinWaves = (MODE == MODE_EXPORT && (F == (F_F32 | F_PASS) || F == (F_BF16 | F_PASS))) ? 7 :
                          (MODE == MODE_SQWA && F == (F_F32 | F_PASS)) ? 5 : 1;

template <int MODE, uint32_t F>
__global__ void __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(kMinWaves<MODE, F>)))
pgq_table_kernel(const TableHeader* __restrict__ hdr,
                                                          const Desc* __restrict__ table,
                                                          const uint32_t* __restrict__ tile_start,
                                                          const uint32_t* __restrict__ tile_desc, KArgs ka)
{
    __shared__ uint32_t hist_all[kWaves][256];
    __shared__ __align__(16) float awq_lds[(F & F_AWQ) ? 2 * kRegCols_F32 : 1];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    uint32_t* hist = hist_all[wave];
    // round 1: the header and this tile's tensor (tile_desc lies inside the workspace whatever
    // it holds); round 2, only for a valid table: that tensor's descriptor.  The owning tensor
    // of the next tile (persistent grids) is fetched one tile ahead.
    uint32_t tile = blockIdx.x;
    const uint64_t magic = hdr->magic;
    const uint64_t checksum = hdr->checksum;
    uint32_t di = tile < ka.n_tiles ? tile_desc[tile] : 0;
    if (magic != kTableMagic || checksum != ka.checksum) {
        if (threadIdx.x == 0 && ka.status) atomicOr(ka.status, PGQ_DEV_STALE_TABLE);
        return;
    }
    uint32_t st = 0;
    while (tile < ka.n_tiles) {
        const uint32_t next = tile + gridDim.x;
        const uint32_t ndi = next < ka.n_tiles ? tile_desc[next] : 0;
        const uint32_t first = tile_start[di];
        const Desc d = fetch_desc<MODE, F>(table + di);
        const int64_t trows = (int64_t)d.tile_rows * (MODE == MODE_TSEL ? ka.tsel_group : 1);
        do_tile<MODE, F>(d, (int64_t)(tile - first) * trows, wave, lane, hist, awq_lds, ka, st);
        tile = next;
        di = ndi;
    }
    st = wave_or(st);
    if (st && lane == 0 && ka.status) atomicOr(ka.status, st);
}

// Final pick of the whole-tensor selects: workgroup i, when tensor i has a per-tensor scale,
// derives its last digit from the histograms (or takes the absmax), stores the key for the
// quantize pass and zeroes the histograms and the running max for the next call.
__global__ void __launch_bounds__(kBlock) pgq_tensor_pick_kernel(const TableHeader* __restrict__ hdr,
                                                                const Desc* __restrict__ table, KArgs ka)
{
    if (hdr->magic != kTableMagic || hdr->checksum != ka.checksum) return;   // the select pass reported it
    if (blockIdx.x >= hdr->n_desc) return;
    const Desc* dp = table + blockIdx.x;
    if (!(dp->flags & DF_TENSOR) || dp->rows <= 0 || dp->cols <= 0) return;
    GLB TState* S = gp(dp->tstate);
    const int tid = (int)threadIdx.x;
    if (dp->rank_top == 1) {                        // absmax: one pass
        if (tid == 0) {
            S->key = S->kmax;
            S->kmax = 0;
        }
        return;
    }
    if (tid < 64) {
        uint32_t prefix, pmask, rem;
        tensor_prefix(S, (uint32_t)dp->rank_top, 4, tid, prefix, pmask, rem);
        if (tid == 0) S->key = prefix & 0x7FFFFFFFu;
    }
    __syncthreads();                                // the histograms are read before they are cleared
#pragma unroll
    for (int p = 0; p < 4; ++p) S->hist[p][tid] = 0;
}

// Decode of stored codes (the artifact loader): x = code * s, divided by a_j for AWQ tensors --
// the export's own dequant, so the result matches it bit for bit.  Codes are int8, or 6-bit
// fields four per three bytes (store_codes6).  One wavefront per row; lane l takes groups of
// four columns l, l + 64, ...
__global__ void __launch_bounds__(kBlock) pgq_decode_kernel(const uint8_t* __restrict__ codes, int32_t packed,
                                                           int64_t rows, int64_t cols,
                                                           const uint16_t* __restrict__ scales, int32_t per_tensor,
                                                           const uint16_t* __restrict__ awq, float* __restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int64_t nw = (int64_t)gridDim.x * kWaves;
    const int64_t ngroups = (cols + 3) >> 2;
    const int64_t rb = packed ? 3 * ngroups : cols;
    for (int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); row < rows; row += nw) {
        const float s = h2f(gp(scales)[per_tensor ? 0 : row]);
        const GLB uint8_t* crow = gp(codes) + row * rb;
        GLB float* orow = gp(out) + row * cols;
        for (int64_t g = lane; g < ngroups; g += 64) {
            int32_t q[4];
            if (packed) {
                const uint32_t w = (uint32_t)crow[3 * g] | ((uint32_t)crow[3 * g + 1] << 8) |
                                   ((uint32_t)crow[3 * g + 2] << 16);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int32_t f = (int32_t)((w >> (6 * t)) & 0x3Fu);
                    q[t] = f >= 32 ? f - 64 : f;
                }
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) q[t] = 4 * g + t < cols ? (int32_t)(int8_t)crow[4 * g + t] : 0;
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int64_t j = 4 * g + t;
                if (j < cols) {
                    float d = (float)q[t] * s;
                    if (awq) d = d / h2f(gp(awq)[j]);       // correctly rounded divide
                    stnt(orow + j, d);
                }
            }
        }
    }
}

// Single-matrix launches: the descriptor is a kernel argument.
template <int MODE, uint32_t F>
__global__ void __launch_bounds__(kBlock) pgq_single_kernel(const Desc d, KArgs ka)
{
    __shared__ uint32_t hist_all[kWaves][256];
    __shared__ __align__(16) float awq_lds[(F & F_AWQ) ? 2 * kRegCols_F32 : 1];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    uint32_t* hist = hist_all[wave];
    uint32_t st = 0;
    for (uint32_t tile = blockIdx.x; tile < ka.n_tiles; tile += gridDim.x)
        do_tile<MODE, F>(d, (int64_t)tile * d.tile_rows, wave, lane, hist, awq_lds, ka, st);
    st = wave_or(st);
    if (st && lane == 0 && ka.status) atomicOr(ka.status, st);
}

template <int MODE, uint32_t F>
const void* kernel_ptr(bool table)
{
    return table ? reinterpret_cast<const void*>(&pgq_table_kernel<MODE, F>)
                 : reinterpret_cast<const void*>(&pgq_single_kernel<MODE, F>);
}

// Instantiations per mode, leanest first; the last covers every feature.
constexpr uint32_t kExportVariants[] = {F_F32 | F_PASS, F_BF16 | F_PASS, F_F32 | F_PASS | F_AWQ,
                                        F_F32 | F_PASS | F_SEL, F_ALL};
constexpr uint32_t kFqVariants[] = {F_BF16, F_BF16 | F_SEL, F_ALL};
constexpr uint32_t kAvgAll = F_F32 | F_BF16 | F_SCALAR;   // also the whole-tensor select's
constexpr uint32_t kAvgVariants[] = {F_F32, F_BF16, kAvgAll};

// Weight averaging and the whole-tensor select run as grouped launches only.
template <int MODE>
const void* average_kernel(uint32_t v, bool table)
{
    if (!table) return nullptr;
    switch (v) {
    case F_F32: return reinterpret_cast<const void*>(&pgq_table_kernel<MODE, F_F32>);
    case F_BF16: return reinterpret_cast<const void*>(&pgq_table_kernel<MODE, F_BF16>);
    default: return reinterpret_cast<const void*>(&pgq_table_kernel<MODE, kAvgAll>);
    }
}

template <int MODE>
const void* export_like(uint32_t v, bool table)
{
    switch (v) {
    case F_F32 | F_PASS: return kernel_ptr<MODE, F_F32 | F_PASS>(table);
    case F_BF16 | F_PASS: return kernel_ptr<MODE, F_BF16 | F_PASS>(table);
    case F_F32 | F_PASS | F_AWQ: return kernel_ptr<MODE, F_F32 | F_PASS | F_AWQ>(table);
    case F_F32 | F_PASS | F_SEL: return kernel_ptr<MODE, F_F32 | F_PASS | F_SEL>(table);
    default: return kernel_ptr<MODE, F_ALL>(table);
    }
}

const void* pick(int mode, uint32_t need, bool table)
{
    const uint32_t v = variant_of(mode, need);
    switch (mode) {
    case MODE_EXPORT: return export_like<MODE_EXPORT>(v, table);
    case MODE_EXPORT6: return export_like<MODE_EXPORT6>(v, table);
    case MODE_SQWA: return export_like<MODE_SQWA>(v, table);
    case MODE_FQ:
        if (v == F_BF16) return kernel_ptr<MODE_FQ, F_BF16>(table);
        if (v == (F_BF16 | F_SEL)) return kernel_ptr<MODE_FQ, F_BF16 | F_SEL>(table);
        return kernel_ptr<MODE_FQ, F_ALL>(table);
    case MODE_FQ_BWD: return kernel_ptr<MODE_FQ_BWD, F_ALL>(table);
    case MODE_EMA: return average_kernel<MODE_EMA>(v, table);
    case MODE_TSEL: return average_kernel<MODE_TSEL>(v, table);
    case MODE_SWA: return average_kernel<MODE_SWA>(v, table);
    case MODE_DECODE: return table ? reinterpret_cast<const void*>(&pgq_table_kernel<MODE_DECODE, F_F32>) : nullptr;
    default: return nullptr;
    }
}

}  // namespace

uint32_t variant_of(int mode, uint32_t need)
{
    if (mode == MODE_EXPORT || mode == MODE_EXPORT6 || mode == MODE_SQWA) {
        for (uint32_t v : kExportVariants)
            if ((need & ~v) == 0) return v;
    } else if (mode == MODE_FQ) {
        for (uint32_t v : kFqVariants)
            if ((need & ~v) == 0) return v;
    } else if (mode == MODE_EMA || mode == MODE_SWA || mode == MODE_TSEL) {
        for (uint32_t v : kAvgVariants)
            if ((need & ~v) == 0) return v;
        return kAvgAll;
    }
    return F_ALL;
}

namespace {
thread_local hipEvent_t t_start = nullptr;   // pgq_time_next_launch
thread_local hipEvent_t t_stop = nullptr;

hipError_t launch_args(const void* fn, uint32_t grid, void** args, hipStream_t s)
{
    if (t_start || t_stop) {
        hipEvent_t a = t_start, b = t_stop;
        t_start = t_stop = nullptr;
        return hipExtLaunchKernel(fn, dim3(grid), dim3(kBlock), args, 0, s, a, b, 0);
    }
    return hipLaunchKernel(fn, dim3(grid), dim3(kBlock), args, 0, s);
}
}  // namespace

int launch_tensor_pick(const KArgs& ka, uint32_t n_desc, void* stream)
{
    if (n_desc == 0) return (int)hipErrorInvalidValue;
    KArgs copy = ka;
    const TableHeader* hdr = ka.hdr;
    const Desc* table = ka.table;
    void* args[] = {&hdr, &table, &copy};
    return (int)launch_args(reinterpret_cast<const void*>(&pgq_tensor_pick_kernel), n_desc, args,
                            static_cast<hipStream_t>(stream));
}

hipError_t launch_plain(const void* fn, dim3 grid, dim3 block, void** args, void* stream)
{
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (t_start || t_stop) {
        hipEvent_t a = t_start, b = t_stop;
        t_start = t_stop = nullptr;
        return hipExtLaunchKernel(fn, grid, block, args, 0, s, a, b, 0);
    }
    return hipLaunchKernel(fn, grid, block, args, 0, s);
}

int launch_decode(const void* codes, int32_t packed, int64_t rows, int64_t cols, const uint16_t* scales,
                  int32_t per_tensor, const uint16_t* awq, float* out, void* stream)
{
    const uint64_t wg = (uint64_t)((rows + kWaves - 1) / kWaves);
    const uint32_t grid = (uint32_t)std::min<uint64_t>(wg, 1u << 16);
    const uint8_t* c = static_cast<const uint8_t*>(codes);
    void* args[] = {&c, &packed, &rows, &cols, &scales, &per_tensor, &awq, &out};
    return (int)launch_args(reinterpret_cast<const void*>(&pgq_decode_kernel), grid, args,
                            static_cast<hipStream_t>(stream));
}

void take_timing_events(void** start, void** stop)
{
    *start = t_start;
    *stop = t_stop;
    t_start = t_stop = nullptr;
}

void set_timing_events(void* start, void* stop)
{
    t_start = static_cast<hipEvent_t>(start);
    t_stop = static_cast<hipEvent_t>(stop);
}

int launch(int mode, uint32_t need, const KArgs& ka, const Desc* single, uint32_t grid, void* stream)
{
    const void* fn = pick(mode, need, single == nullptr);
    if (!fn || grid == 0) return (int)hipErrorInvalidValue;
    KArgs copy = ka;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (single) {
        Desc d = *single;
        void* args[] = {&d, &copy};
        return (int)launch_args(fn, grid, args, s);
    }
    const TableHeader* hdr = ka.hdr;
    const Desc* table = ka.table;
    const uint32_t* tile_start = ka.tile_start;
    const uint32_t* tile_desc = ka.tile_desc;
    void* args[] = {&hdr, &table, &tile_start, &tile_desc, &copy};
    return (int)launch_args(fn, grid, args, s);
}

int max_resident_blocks(int mode, uint32_t need, bool table, int* per_cu, int* n_cu)
{
    const void* fn = pick(mode, need, table);
    if (!fn) return (int)hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    e = hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return (int)e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, fn, kBlock, 0);
    return (int)e;
}

}  // namespace pgq
