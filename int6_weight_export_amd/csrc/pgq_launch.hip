// pgq_launch.hip -- launch side of libpgq's kernels: the choice of instantiation, timing events,
// and the small non-template kernels (the whole-tensor pick, the single-tensor decode).
#include "pgq_kern.h"

namespace pgq {
namespace {

// Final pick of the whole-tensor selects: workgroup i, when tensor i has a per-tensor scale,
// finds its clip key -- the R-th largest of its candidate keys (DF_CAND), the last digit from the
// radix passes' histograms, or the absmax -- stores it for the quantize pass and zeroes the
// histograms and the running max for the next call.
constexpr uint32_t kPickBuf = 2048;           // candidates ranked directly in LDS
constexpr int kPickThreads = 1024;            // threads of a pick workgroup
constexpr int kPickWaves = kPickThreads / 64;
constexpr int kPickGroups = 8;                // four-slot groups a thread keeps in registers

// DF_CAND: the R-th largest of the candidate keys, which sit in ccap slots per candidate tile
// (a multiple of 4), the first count[tile] of them valid.  The workgroup loads them once into
// registers (when they fit; otherwise every pass streams them), each thread keeping the maximum
// of its share; a lower bound on the R-th largest of those thread maxima (wg_lower_bound) bounds
// the answer from below, so only the candidates at or above it can be it: they are gathered
// (usually a few hundred) and each is ranked against all of them.  More than kPickBuf of them
// (heavy ties) fall back to a radix select over the valid candidates.
__device__ __forceinline__ void cand_pick(const Desc* dp, GLB TState* S, uint32_t* sl, uint32_t* buf)
{
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const uint32_t R = (uint32_t)dp->rank_top;
    const uint32_t cap = (uint32_t)dp->ccap;
    const uint32_t ntiles = (uint32_t)((dp->rows + dp->crows - 1) / dp->crows);
    const GLB uint32_t* cand = gp(dp->cand);
    const GLB uint32_t* count = cand + (size_t)ntiles * cap;
    const uint32_t slots = ntiles * cap;
    const bool held = slots <= 4u * kPickThreads * kPickGroups;
    u32x4 v[kPickGroups];
    uint32_t ok = 0;                                 // bit 4 g + e: v[g][e] is a valid candidate
    if (held) {
#pragma unroll
        for (int g = 0; g < kPickGroups; ++g) {
            const uint32_t s = 4u * ((uint32_t)tid + (uint32_t)g * kPickThreads);
            if (s < slots) {
                v[g] = *reinterpret_cast<const GLB u32x4*>(cand + s);
                const uint32_t tile = s / cap;
                const uint32_t i = s - tile * cap;
                const uint32_t n = count[tile];
#pragma unroll
                for (int e = 0; e < 4; ++e) ok |= (i + (uint32_t)e < n ? 1u : 0u) << (4 * g + e);
            }
        }
    }
    // every valid candidate: from the registers, or streamed in four-slot groups
    auto each = [&](auto&& f) PGQ_AI {
        if (held) {
#pragma unroll
            for (int g = 0; g < kPickGroups; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if ((ok >> (4 * g + e)) & 1u) f(v[g][e]);
            return;
        }
#pragma unroll 4
        for (uint32_t s = 4u * (uint32_t)tid; s < slots; s += 4u * kPickThreads) {
            const u32x4 w = *reinterpret_cast<const GLB u32x4*>(cand + s);
            const uint32_t tile = s / cap;
            const uint32_t n = count[tile];
            const uint32_t i = s - tile * cap;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (i + (uint32_t)e < n) f(w[e]);
        }
    };
    uint32_t lm = 0;
    each([&](uint32_t k) PGQ_AI { lm = max(lm, k + 1u); });
    const uint32_t t1 = wg_lower_bound<kPickWaves>(lm, R, wave, lane, sl);
    if (tid == 0) sl[300] = 0;
    __syncthreads();
    each([&](uint32_t k) PGQ_AI {
        if (k + 1u >= t1) {
            const uint32_t slot = atomicAdd(&sl[300], 1u);
            if (slot < kPickBuf) buf[slot] = k;
        }
    });
    __syncthreads();
    const uint32_t C = sl[300];
    if (C <= kPickBuf) {
        for (uint32_t q = (uint32_t)tid; q < C; q += kPickThreads) {
            const uint32_t x = buf[q];
            uint32_t gt = 0, ge = 0;
            for (uint32_t u = 0; u < C; ++u) {
                gt += buf[u] > x ? 1u : 0u;
                ge += buf[u] >= x ? 1u : 0u;
            }
            if (gt < R && R <= ge) S->key = x;       // the same value from every finder
        }
        return;
    }
    // radix select over the valid candidates, digits of bits 30..23, 22..15, 14..7, 6..0
    uint32_t prefix = 0, pmask = 0, rem = R;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = pass == 0 ? 23 : pass == 1 ? 15 : pass == 2 ? 7 : 0;
        if (tid < 256) buf[tid] = 0;
        __syncthreads();
        each([&](uint32_t k) PGQ_AI {
            if ((k & pmask) == prefix) atomicAdd(&buf[(k >> shift) & 0xFFu], 1u);
        });
        __syncthreads();
        if (wave == 0) {
            uint32_t digit, above;
            radix_digit(buf, rem, lane, digit, above);
            if (lane == 0) { sl[301] = digit; sl[302] = above; }
        }
        __syncthreads();
        rem -= sl[302];
        prefix |= sl[301] << shift;
        pmask |= 0xFFu << shift;
        __syncthreads();
    }
    if (tid == 0) S->key = prefix;
}

__global__ void __launch_bounds__(kPickThreads) pgq_tensor_pick_kernel(const TableHeader* __restrict__ hdr,
                                                                      const Desc* __restrict__ table, KArgs ka)
{
    __shared__ uint32_t sl[320];
    __shared__ uint32_t buf[kPickBuf];
    if (hdr->magic != kTableMagic || hdr->checksum != ka.checksum) return;   // the select pass reported it
    if (blockIdx.x >= hdr->n_desc) return;
    const Desc* dp = table + blockIdx.x;
    if (!(dp->flags & DF_TENSOR) || dp->rows <= 0 || dp->cols <= 0) return;
    GLB TState* S = gp(dp->tstate);
    const int tid = (int)threadIdx.x;
    if (dp->flags & DF_CAND) {
        cand_pick(dp, S, sl, buf);
        return;
    }
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
    if (tid < 256) {
#pragma unroll
        for (int p = 0; p < 4; ++p) S->hist[p][tid] = 0;
    }
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

const void* pick(int mode, uint32_t need, bool table)
{
    const uint32_t v = variant_of(mode, need);
    switch (mode) {
#define PGQ_EXPORT_LIKE(m)                                                    \
    if (is_lean_variant(v)) return kernels_##m(v, table);                     \
    if (v == (F_F32 | F_PASS | F_SEL)) return kernels_##m##_sel(table);        \
    return table ? kernels_##m##_all_table() : kernels_##m##_all_single();
    case MODE_EXPORT: PGQ_EXPORT_LIKE(export)
    case MODE_EXPORT6: PGQ_EXPORT_LIKE(export6)
    case MODE_SQWA: PGQ_EXPORT_LIKE(sqwa)
#undef PGQ_EXPORT_LIKE
    case MODE_FQ:
    case MODE_FQ_BWD: return kernels_fq(mode, v, table);
    case MODE_EMA:
    case MODE_TSEL:
    case MODE_TCAND:
    case MODE_SWA:
    case MODE_DECODE: return kernels_avg(mode, v, table);
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
    } else if (mode == MODE_EMA || mode == MODE_SWA || mode == MODE_TSEL || mode == MODE_TCAND) {
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
    return (int)launch_plain(reinterpret_cast<const void*>(&pgq_tensor_pick_kernel), dim3(n_desc),
                             dim3(kPickThreads), args, stream);
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


}  // namespace pgq
