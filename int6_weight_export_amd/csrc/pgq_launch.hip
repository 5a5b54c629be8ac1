// pgq_launch.hip -- launch side of libpgq's kernels: the choice of instantiation, timing events,
// and the small non-template kernels (the whole-tensor pick, the single-tensor decode).
#include "pgq_kern.h"

namespace pgq {
namespace {

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
