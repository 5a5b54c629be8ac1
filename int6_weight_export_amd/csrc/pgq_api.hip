// pgq_api.hip -- host layer of libpgq: argument checks, export planning, descriptor
// tables and launches behind the C ABI declared in include/pgq.h.
//
// Argument errors return before anything is enqueued.  Grouped calls write one table
// (header + per-tensor descriptors + row tiles) into the caller's workspace with one
// host-to-device copy on the caller's stream, unless PGQ_TABLE_RESIDENT says the same
// table is already there; the kernels verify its checksum either way.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "pgq_desc.h"
#include "../../include/pgq.h"

using namespace pgq;

namespace {

// Launch geometry, fixed from measurements on MI355X.
constexpr int kGroupsPerWave = 1;       // row groups per wavefront in one tile (a tile is
                                        // kWaves * rgroup * groups rows of a tensor)
constexpr int kAwqGroupsPerWave = 2;    // the same for tensors with AWQ multipliers: the workgroup
                                        // builds the multiplier table once per tile
constexpr int kSelGroup = 3;            // export tiles per workgroup of a radix select pass
constexpr int kFlatMaxLoads = 5;        // wave-wide loads of one flat run (STE: 8 registers each)
constexpr uint32_t kCandMaxRank = 256;  // candidate select up to this rank from the top

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool qparams_ok(const pgq_qparams& q)
{
    return q.bits >= 2 && q.bits <= 8 && q.pct_den > 0 && q.pct_num <= q.pct_den;
}

// The clip is the k-th smallest |x| with k = ceil(num * n / den) in [1, n]; kernels use
// its rank from the top, n - k + 1.
int64_t rank_top(int64_t n, uint32_t num, uint32_t den)
{
    if (n <= 0) return 1;
    unsigned __int128 p = (unsigned __int128)num * (unsigned __int128)n;
    int64_t k = (int64_t)((p + den - 1) / den);
    k = std::min(std::max<int64_t>(k, 1), n);
    return n - k + 1;
}

// 64-bit hash of a table (multiply-xorshift over 8-byte words; n is a multiple of 8).
uint64_t table_hash(const void* data, size_t n, uint64_t h)
{
    const uint8_t* p = static_cast<const uint8_t*>(data);
    for (size_t i = 0; i < n; i += 8) {
        uint64_t w = 0;
        memcpy(&w, p + i, std::min<size_t>(8, n - i));
        h = (h ^ w) * 0x9E3779B97F4A7C15ull;
        h ^= h >> 29;
    }
    return h;
}

size_t esize(int32_t dt) { return dt == PGQ_F32 ? 4 : 2; }
bool weight_dtype_ok(int32_t dt) { return dt == PGQ_F32 || dt == PGQ_BF16 || dt == PGQ_F16; }
int32_t in_of(int32_t dt) { return dt == PGQ_F32 ? IN_F32 : dt == PGQ_F16 ? IN_F16 : IN_BF16; }

bool shape_ok(int64_t rows, int64_t cols, int64_t ld)
{
    if (rows < 0 || cols < 0 || ld < cols) return false;
    if (cols > ((int64_t)1 << 29) - 64) return false;           // a row's byte offsets fit in 32 bits
    if (rows > ((int64_t)1 << 32) - 1) return false;            // tile row origins are 32-bit
    return true;
}

// Vector (16-byte) path: every stream of this tensor is aligned to its vector width.
void set_vec_flag(Desc& d)
{
    const int vec = d.in_dtype == IN_F32 ? 4 : 8;
    const size_t ein = d.in_dtype == IN_F32 ? 4 : 2;
    bool ok = d.cols % vec == 0 && d.ld % vec == 0 && aligned(d.w, 16);
    const size_t dqe = d.dq_dtype == IN_F32 ? 4 : 2;
    ok = ok && (!d.codes || (d.flags & DF_PACK6) || aligned(d.codes, vec));
    ok = ok && (!d.dq || aligned(d.dq, std::min<size_t>(16, vec * dqe)));
    ok = ok && (!d.awq_s || aligned(d.awq_s, 16));
    ok = ok && (!d.awq_out || aligned(d.awq_out, vec * 2));
    ok = ok && (!d.f16_out || aligned(d.f16_out, vec * 2));
    ok = ok && (!d.mean || aligned(d.mean, 16));
    ok = ok && (!d.grad || aligned(d.grad, 16));
    ok = ok && (!d.grad_out || aligned(d.grad_out, 16));
    (void)ein;
    d.flags = (d.flags & ~(uint32_t)DF_VEC) | (ok ? (uint32_t)DF_VEC : 0u);
}

// Kernel features a tensor needs (see F_* in pgq_desc.h).
uint32_t features_of(const Desc& d)
{
    if (d.rows <= 0 || d.cols <= 0) return 0;
    uint32_t f = d.in_dtype == IN_F32 ? F_F32 : d.in_dtype == IN_F16 ? F_F16 : F_BF16;
    const bool vec = (d.flags & DF_VEC) != 0;
    if (!vec) f |= F_SCALAR;
    if (d.kind == KIND_F16) return f | F_PASS;
    if (d.awq_s) f |= F_AWQ;
    if (d.rank_top > 1 && !(d.flags & DF_TENSOR)) f |= F_SEL;
    const int64_t reg_cols = !vec ? kRegCols_Scalar : (d.in_dtype == IN_F32 ? kRegCols_F32 : kRegCols_BF16);
    if (d.cols > reg_cols) f |= F_LONG;
    return f;
}

// Weight averaging reads only the input dtype and the vector flag.
uint32_t features_avg(const Desc& d)
{
    if (d.rows <= 0 || d.cols <= 0) return 0;
    return (d.in_dtype == IN_F32 ? F_F32 : d.in_dtype == IN_F16 ? F_F16 : F_BF16) |
           ((d.flags & DF_VEC) ? 0u : F_SCALAR);
}

Desc blank_desc()
{
    Desc d;
    memset(&d, 0, sizeof(d));
    d.rank_top = 1;
    d.rgroup = 1;
    d.tile_rows = kWaves;
    return d;
}

// One workgroup per tile: the hardware dispatcher balances the load (a persistent grid striding
// over the tiles measured ~10% slower).
uint32_t grid_for(uint32_t n_tiles) { return std::max<uint32_t>(1, n_tiles); }

// Workspace layout of a grouped call: header | descriptors | first tile per tensor | tensor per
// tile | (per-tensor scales) first tile per tensor and tensor per tile of the radix select passes
// and of the candidate pass | one TState per tensor | candidate keys.  The parts after the main
// table are uploaded only when a call selects (the TStates start at zero); the candidate region
// is never uploaded.
struct TableLayout {
    size_t desc_off, start_off, tdesc_off, end_main, start2_off, tdesc2_off, start3_off, tdesc3_off, state_off,
        state_end, cand_off, end;
};

TableLayout table_layout(size_t n_desc, uint64_t n_tiles, uint64_t cand_words)
{
    TableLayout L;
    const int64_t starts = align_up((int64_t)((n_desc + 1) * sizeof(uint32_t)), 64);
    const int64_t tiles = align_up((int64_t)(n_tiles * sizeof(uint32_t)), 64);
    L.desc_off = sizeof(TableHeader);
    L.start_off = L.desc_off + align_up((int64_t)(n_desc * sizeof(Desc)), 64);
    L.tdesc_off = L.start_off + starts;
    L.end_main = L.tdesc_off + align_up((int64_t)(n_tiles * sizeof(uint32_t)), 8);
    L.start2_off = align_up((int64_t)L.end_main, 64);
    L.tdesc2_off = L.start2_off + starts;
    L.start3_off = L.tdesc2_off + tiles;
    L.tdesc3_off = L.start3_off + starts;
    L.state_off = L.tdesc3_off + tiles;
    L.state_end = L.state_off + n_desc * sizeof(TState);
    L.cand_off = align_up((int64_t)L.state_end, 256);
    L.end = L.cand_off + cand_words * sizeof(uint32_t);
    return L;
}

size_t table_bytes(size_t n_desc, uint64_t n_tiles, uint64_t cand_words = 0)
{
    return table_layout(n_desc, n_tiles, cand_words).end;
}

// Candidate select geometry: a lane of a candidate tile holds kCandKeys keys, and one row gives
// it ceil(cols / (64 vec)) slots of vec elements; rows per wavefront, 0 when a row does not fit.
int cand_rows_per_wave(int64_t cols, int vec)
{
    const int64_t per_row = ((cols / vec + 63) / 64) * vec;
    return per_row > 32 ? 0 : (int)(32 / per_row);
}

// Keys a candidate tile may append: twice the rank plus slack (a tile appends every key at or
// above its bound, about the rank for independent values; beyond this it appends its exact
// rank_top largest instead).
uint32_t cand_cap(int64_t rank) { return (uint32_t)((2 * rank + 32 + 3) & ~(int64_t)3); }

// Words of one tensor's candidate region: ccap slots per tile, then one count per tile.
uint64_t cand_region_words(uint64_t tiles, uint32_t ccap) { return (uint64_t)align_up((int64_t)(tiles * ccap + tiles), 16); }

// Candidate words a per-tensor tensor needs, whichever load path (vector or element-wise) its
// export takes; 0 when it uses the radix select.
uint64_t cand_words_bound(int64_t rows, int64_t cols, int32_t dtype, int64_t rank)
{
    if (rank > (int64_t)kCandMaxRank || rows <= 0 || cols <= 0) return 0;
    const int vec = dtype == PGQ_F32 ? 4 : 8;
    int rpw = cand_rows_per_wave(cols, 1);
    if (cols % vec == 0) {
        const int rv = cand_rows_per_wave(cols, vec);
        rpw = std::min(rpw, rv);
    }
    if (rpw <= 0) return 0;
    const int64_t tiles = (rows + (int64_t)kWaves * rpw - 1) / ((int64_t)kWaves * rpw);
    return cand_region_words((uint64_t)tiles, cand_cap(rank));
}

// Rows a wavefront loads together: as many as the register tile holds (a power of two), and
// the exact chunk count per lane of a row on the vector path.
void set_grouping(Desc& d, int mode)
{
    int R = 1;
    d.nch = 0;
    if (mode != MODE_FQ_BWD && mode != MODE_EMA && mode != MODE_SWA && mode != MODE_DECODE && d.kind != KIND_F16 &&
        d.cols > 0) {
        const bool vec = (d.flags & DF_VEC) != 0;
        const int64_t nchunk = vec ? d.cols / (d.in_dtype == IN_F32 ? 4 : 8) : d.cols;
        const int ncht = vec ? (d.in_dtype == IN_F32 ? 8 : 4) : 16;
        const int64_t nch = (nchunk + 63) / 64;
        if (nch <= ncht) {
            if (vec) d.nch = (int32_t)nch;
            int p2 = 1;
            while (p2 < nch) p2 <<= 1;
            // measured: STE rows (bf16, two input streams) gain from two rows per wavefront,
            // export and SQWA rows from one
            const int cap = mode == MODE_FQ ? 2 : 1;
            R = std::min(std::min(ncht / p2, 8), cap);
            int r2 = 1;
            while (r2 * 2 <= R) r2 *= 2;
            R = r2;
        }
    }
    // Flat runs (DF_FLAT): dense bf16 rows of K = cols / 8 chunks, 64 < K < 5 * 64 and K not a
    // multiple of 64, absmax per row, no AWQ.  R rows are read as one run of IT = ceil(R K / 64)
    // wave-wide loads; take the R <= 8 with IT <= kFlatMaxLoads (STE; one fewer for exports, whose
    // kernels keep more waves per SIMD) that uses the loads best, when that beats ceil(K / 64)
    // loads per row by a margin.
    d.flags &= ~DF_FLAT;
    if ((mode == MODE_FQ || mode == MODE_EXPORT) && (d.flags & DF_VEC) && d.in_dtype == IN_BF16 &&
        d.kind != KIND_F16 && !d.awq_s && !(d.flags & DF_TENSOR) && d.rank_top <= 1 && d.ld == d.cols &&
        d.cols % 8 == 0) {
        const int64_t K = d.cols / 8;
        const int max_loads = mode == MODE_FQ ? kFlatMaxLoads : kFlatMaxLoads - 1;
        if (K > 64 && K % 64 != 0 && K < 64 * max_loads) {
            const double row_use = (double)K / (64.0 * (double)((K + 63) / 64));
            int best_r = 0, best_it = 0;
            double best_use = row_use + 0.05;
            for (int r = 1; r <= 8; ++r) {
                const int64_t it = (r * K + 63) / 64;
                if (it > max_loads) break;
                const double use = (double)(r * K) / (64.0 * (double)it);
                if (use > best_use) { best_use = use; best_r = r; best_it = (int)it; }
            }
            if (best_r > 0) {
                d.flags |= DF_FLAT;
                R = best_r;
                d.nch = best_it;
            }
        }
    }
    // decode rows are short (a few KB of output each): two rows per wavefront halve the tiles and
    // their per-workgroup start-up (measured 23.2 -> 20.0 us on the 9-layer artifact); four or
    // eight rows per wavefront, one after another, ran slower
    if (mode == MODE_DECODE) R = 2;
    d.rgroup = R;
    const bool awq_tile = d.awq_s && d.kind != KIND_F16 && mode != MODE_FQ && mode != MODE_FQ_BWD;
    d.tile_rows = kWaves * R * std::max(kGroupsPerWave, awq_tile ? kAwqGroupsPerWave : 1);
}

// Upper bound on the tiles of a tensor (group size 1), for sizing workspaces before the
// output pointers, and so the vector path and group size, are known.
uint64_t max_tiles_for(int64_t rows, int64_t cols)
{
    if (rows <= 0 || cols <= 0) return 0;
    const int64_t tr = (int64_t)kWaves * kGroupsPerWave;
    return (uint64_t)((rows + tr - 1) / tr);
}

uint64_t tiles_for(const Desc& d)
{
    if (d.rows <= 0 || d.cols <= 0) return 0;
    return (uint64_t)((d.rows + d.tile_rows - 1) / d.tile_rows);
}

// The HIP error behind this thread's latest PGQ_ERR_HIP (pgq_last_error).
thread_local hipError_t t_last_hip = hipSuccess;

pgq_status hip_failed(hipError_t e)
{
    t_last_hip = e;
    return PGQ_ERR_HIP;
}

// Build the table on the host, upload it (unless resident) and launch one grouped kernel.
pgq_status run_grouped(int mode, const std::vector<Desc>& descs_in, void* ws, size_t ws_bytes,
                       uint32_t flags, uint32_t* dev_status, int sqwa_k, int fq_mode, void* stream,
                       int avg_init = 0, float avg_d = 0.0f, float avg_c = 0.0f)
{
    if (mode == MODE_EXPORT)
        for (const Desc& d : descs_in)
            if (d.flags & DF_PACK6) mode = MODE_EXPORT6;
    // Longest tiles first: workgroups start in tile order, so the launch ends on the shortest
    // tiles and its tail is short.  (The tensors' order has no other meaning to the kernel.)
    std::vector<Desc> descs(descs_in);
    std::stable_sort(descs.begin(), descs.end(), [](const Desc& a, const Desc& b) {
        return (int64_t)a.tile_rows * a.cols > (int64_t)b.tile_rows * b.cols;
    });
    const size_t n = descs.size();
    std::vector<uint32_t> start(n + 1, 0);
    uint64_t total = 0;
    for (size_t i = 0; i < n; ++i) {
        start[i] = (uint32_t)total;
        total += tiles_for(descs[i]);
        if (total > 0xFFFFFFF0ull) return PGQ_ERR_SHAPE;
    }
    start[n] = (uint32_t)total;
    if (total == 0) return PGQ_OK;
    // per-tensor scales (only an export selects; a decode's DF_TENSOR just means "scale 0 for
    // every row"): the clip of a tensor with rank_top <= kCandMaxRank and rows that fit a
    // candidate tile comes from the one-read candidate pass, any other from the radix passes
    // (kSelGroup export tiles per workgroup)
    const TableLayout L0 = table_layout(n, total, 0);
    std::vector<uint32_t> start2(n + 1, 0), start3(n + 1, 0);
    uint64_t total2 = 0, total3 = 0, cand_words = 0;
    int passes = 0;
    const bool selects = mode == MODE_EXPORT || mode == MODE_EXPORT6;
    for (size_t i = 0; i < n; ++i) {
        start2[i] = (uint32_t)total2;
        start3[i] = (uint32_t)total3;
        Desc& d = descs[i];
        if (selects && (d.flags & DF_TENSOR) && d.rows > 0 && d.cols > 0) {
            if (!d.w) return PGQ_ERR_NULL;                          // the select reads the weights
            d.tstate = reinterpret_cast<TState*>(static_cast<uint8_t*>(ws) + L0.state_off) + i;
            const bool vec = (d.flags & DF_VEC) != 0;
            const int rpw = cand_rows_per_wave(d.cols, vec ? (d.in_dtype == IN_F32 ? 4 : 8) : 1);
            if (d.rank_top <= (int64_t)kCandMaxRank && rpw > 0) {
                d.flags |= DF_CAND;
                d.crows = kWaves * rpw;
                d.ccap = (int32_t)cand_cap(d.rank_top);
                const uint64_t ct = (uint64_t)((d.rows + d.crows - 1) / d.crows);
                d.cand = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + L0.cand_off) + cand_words;
                cand_words += cand_region_words(ct, (uint32_t)d.ccap);
                total3 += ct;
            } else {
                total2 += (tiles_for(d) + kSelGroup - 1) / kSelGroup;
                passes = std::max(passes, d.rank_top > 1 ? 4 : 1);
            }
        }
    }
    start2[n] = (uint32_t)total2;
    start3[n] = (uint32_t)total3;
    const bool select = passes > 0 || total3 > 0;
    const TableLayout L = table_layout(n, total, cand_words);
    const size_t need = select ? L.end : L.end_main;            // bytes the call uses
    const size_t upload = select ? L.state_end : L.end_main;    // bytes the host writes
    if (!ws) return PGQ_ERR_WORKSPACE;
    if (ws_bytes < need) return PGQ_ERR_WORKSPACE;
    if (!aligned(ws, 64)) return PGQ_ERR_ALIGN;

    // The checksum covers the descriptors and the tile prefixes (the per-tile tensor indices are
    // functions of them), so a call on a resident table hashes ~n * 180 bytes and builds nothing
    // else.
    uint64_t h = table_hash(descs.data(), n * sizeof(Desc), 0x243F6A8885A308D3ull ^ (uint64_t)mode);
    h = table_hash(start.data(), (n + 1) * sizeof(uint32_t), h);
    h = table_hash(&total, 8, h);
    if (select) {
        h = table_hash(start2.data(), (n + 1) * sizeof(uint32_t), h);
        h = table_hash(start3.data(), (n + 1) * sizeof(uint32_t), h);
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!(flags & PGQ_TABLE_RESIDENT)) {
        std::vector<uint64_t> buf8((upload + 7) / 8, 0);
        uint8_t* buf = reinterpret_cast<uint8_t*>(buf8.data());
        TableHeader* hdr = reinterpret_cast<TableHeader*>(buf);
        memcpy(buf + L.desc_off, descs.data(), n * sizeof(Desc));
        memcpy(buf + L.start_off, start.data(), (n + 1) * sizeof(uint32_t));
        uint32_t* tdesc = reinterpret_cast<uint32_t*>(buf + L.tdesc_off);
        for (size_t i = 0; i < n; ++i)
            for (uint32_t t = start[i]; t < start[i + 1]; ++t) tdesc[t] = (uint32_t)i;
        if (select) {                                      // the TStates start at zero
            memcpy(buf + L.start2_off, start2.data(), (n + 1) * sizeof(uint32_t));
            memcpy(buf + L.start3_off, start3.data(), (n + 1) * sizeof(uint32_t));
            uint32_t* tdesc2 = reinterpret_cast<uint32_t*>(buf + L.tdesc2_off);
            uint32_t* tdesc3 = reinterpret_cast<uint32_t*>(buf + L.tdesc3_off);
            for (size_t i = 0; i < n; ++i) {
                for (uint32_t t = start2[i]; t < start2[i + 1]; ++t) tdesc2[t] = (uint32_t)i;
                for (uint32_t t = start3[i]; t < start3[i + 1]; ++t) tdesc3[t] = (uint32_t)i;
            }
        }
        hdr->magic = kTableMagic;
        hdr->checksum = h;
        hdr->n_desc = (uint32_t)n;
        hdr->n_tiles = (uint32_t)total;
        // A pageable source is staged by the runtime before this call returns.
        const hipError_t e = hipMemcpyAsync(ws, buf, upload, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_failed(e);
    }
    const uint8_t* base = static_cast<const uint8_t*>(ws);
    KArgs ka;
    memset(&ka, 0, sizeof(ka));
    ka.hdr = reinterpret_cast<const TableHeader*>(base);
    ka.table = reinterpret_cast<const Desc*>(base + L.desc_off);
    ka.checksum = h;
    ka.status = dev_status;
    ka.sqwa_k = sqwa_k;
    ka.fq_mode = fq_mode;
    ka.avg_init = avg_init;
    ka.avg_d = avg_d;
    ka.avg_c = avg_c;
    void *ev_start = nullptr, *ev_stop = nullptr;
    take_timing_events(&ev_start, &ev_stop);
    // the whole-tensor clip select -- the candidate pass and / or one launch per radix digit --
    // and the final pick, then the main launch
    if (select) {
        uint32_t fc = 0, fr = 0;
        for (const Desc& d : descs)
            if (d.flags & DF_TENSOR) ((d.flags & DF_CAND) ? fc : fr) |= features_avg(d);
        if (total3) {
            KArgs k3 = ka;
            k3.tile_start = reinterpret_cast<const uint32_t*>(base + L.start3_off);
            k3.tile_desc = reinterpret_cast<const uint32_t*>(base + L.tdesc3_off);
            k3.n_tiles = (uint32_t)total3;
            set_timing_events(ev_start, nullptr);
            ev_start = nullptr;
            if (const int e = launch(MODE_TCAND, fc, k3, nullptr, grid_for(k3.n_tiles), stream))
                return hip_failed((hipError_t)e);
        }
        KArgs k2 = ka;
        k2.tile_start = reinterpret_cast<const uint32_t*>(base + L.start2_off);
        k2.tile_desc = reinterpret_cast<const uint32_t*>(base + L.tdesc2_off);
        k2.n_tiles = (uint32_t)total2;
        k2.tsel_group = kSelGroup;
        for (int p = 0; p < passes; ++p) {
            k2.tsel_pass = p;
            set_timing_events(ev_start, nullptr);
            ev_start = nullptr;
            if (const int e = launch(MODE_TSEL, fr, k2, nullptr, grid_for(k2.n_tiles), stream))
                return hip_failed((hipError_t)e);
        }
        if (const int e = launch_tensor_pick(k2, (uint32_t)n, stream)) return hip_failed((hipError_t)e);
    }
    ka.tile_start = reinterpret_cast<const uint32_t*>(base + L.start_off);
    ka.tile_desc = reinterpret_cast<const uint32_t*>(base + L.tdesc_off);
    ka.n_tiles = (uint32_t)total;
    const bool averaging = mode == MODE_EMA || mode == MODE_SWA;
    uint32_t feats = 0;
    for (const Desc& d : descs) feats |= averaging ? features_avg(d) : features_of(d);
    const uint32_t grid = grid_for(ka.n_tiles);
    set_timing_events(ev_start, ev_stop);
    if (const int e = launch(mode, feats, ka, nullptr, grid, stream)) return hip_failed((hipError_t)e);
    if (const hipError_t e = hipGetLastError()) return hip_failed(e);
    return PGQ_OK;
}

pgq_status run_single(int mode, const Desc& d, uint32_t* dev_status, int sqwa_k, int fq_mode, void* stream)
{
    if (d.rows <= 0 || d.cols <= 0) return PGQ_OK;
    KArgs ka;
    memset(&ka, 0, sizeof(ka));
    ka.status = dev_status;
    const uint64_t nt = tiles_for(d);
    if (nt > 0xFFFFFFFFull) return PGQ_ERR_SHAPE;
    ka.n_tiles = (uint32_t)nt;
    ka.sqwa_k = sqwa_k;
    ka.fq_mode = fq_mode;
    const uint32_t need = features_of(d);
    const uint32_t grid = grid_for(ka.n_tiles);
    if (const int e = launch(mode, need, ka, &d, grid, stream)) return hip_failed((hipError_t)e);
    if (const hipError_t e = hipGetLastError()) return hip_failed(e);
    return PGQ_OK;
}

bool name_matches(const char* name, const pgq_policy* pol)
{
    const char* nm = name ? name : "";
    for (int32_t i = 0; i < pol->n_patterns; ++i) {
        const char* p = pol->int8_patterns[i];
        if (p && *p && strstr(nm, p)) return true;
    }
    return false;
}

pgq_status check_tensor_in(const pgq_tensor_in& t)
{
    if (!shape_ok(t.rows, t.cols, t.ld)) return PGQ_ERR_SHAPE;
    if (!weight_dtype_ok(t.dtype)) return PGQ_ERR_DTYPE;
    if (t.rows > 0 && t.cols > 0 && !t.w) return PGQ_ERR_NULL;
    if (t.w && !aligned(t.w, esize(t.dtype))) return PGQ_ERR_ALIGN;
    if (t.awq_s && !aligned(t.awq_s, 4)) return PGQ_ERR_ALIGN;
    return PGQ_OK;
}

// Descriptors of a weight-averaging call: weights in, fp32 state rows x cols (dense) in place.
pgq_status average_descs(const pgq_tensor_in* w, int32_t n, float* const* state, int mode,
                         std::vector<Desc>& descs)
{
    descs.assign((size_t)n, blank_desc());
    for (int32_t i = 0; i < n; ++i) {
        const pgq_status st = check_tensor_in(w[i]);
        if (st != PGQ_OK) return st;
        if (w[i].awq_s) return PGQ_ERR_PARAM;
        Desc& d = descs[i];
        d.w = w[i].w;
        d.in_dtype = in_of(w[i].dtype);
        d.rows = w[i].rows;
        d.cols = w[i].cols;
        d.ld = w[i].ld;
        if (d.rows > 0 && d.cols > 0) {
            if (!state[i]) return PGQ_ERR_NULL;
            if (!aligned(state[i], 4)) return PGQ_ERR_ALIGN;
        }
        d.mean = state[i];
        set_vec_flag(d);
        set_grouping(d, mode);
    }
    return PGQ_OK;
}

pgq_status check_plan_entry(const pgq_tensor_plan& p)
{
    if (p.kind == PGQ_KIND_F16) return PGQ_OK;
    if (p.kind < 2 || p.kind > 8 || p.qp.bits != p.kind || !qparams_ok(p.qp)) return PGQ_ERR_PARAM;
    if (p.per_tensor != 0 && p.per_tensor != 1) return PGQ_ERR_PARAM;
    if (p.packed != 0 && (p.packed != 1 || p.kind != 6)) return PGQ_ERR_PARAM;
    return PGQ_OK;
}

// Descriptor of one export / SQWA tensor from its input and plan entry.
pgq_status export_desc(const pgq_tensor_in& t, const pgq_tensor_plan& p, uint8_t* arena, Desc& d)
{
    d = blank_desc();
    d.w = t.w;
    d.rows = t.rows;
    d.cols = t.cols;
    d.ld = t.ld;
    d.in_dtype = in_of(t.dtype);
    d.dq_dtype = IN_F32;
    const int64_t numel = t.rows * t.cols;
    if (p.kind == PGQ_KIND_F16) {
        d.kind = KIND_F16;
        if (arena && numel > 0) {
            if (p.f16_off < 0) return PGQ_ERR_PARAM;
            d.f16_out = reinterpret_cast<uint16_t*>(arena + p.f16_off);
        }
    } else {
        d.kind = p.kind;
        d.Q = (1 << (p.kind - 1)) - 1;
        if (p.per_tensor) {
            if (p.has_awq) return PGQ_ERR_PARAM;
            d.flags |= DF_TENSOR;
            if (numel >= (int64_t(1) << 32)) return PGQ_ERR_SHAPE;
            d.rank_top = numel > 0 ? rank_top(numel, p.qp.pct_num, p.qp.pct_den) : 1;
        } else {
            d.rank_top = rank_top(t.cols, p.qp.pct_num, p.qp.pct_den);
        }
        if (arena && numel > 0) {
            if (p.codes_off < 0 || p.scales_off < 0) return PGQ_ERR_PARAM;
            d.codes = reinterpret_cast<int8_t*>(arena + p.codes_off);
            d.scales = reinterpret_cast<uint16_t*>(arena + p.scales_off);
            if (p.packed) d.flags |= DF_PACK6;
        }
        if (p.has_awq) {
            if (!t.awq_s) return PGQ_ERR_NULL;
            d.awq_s = t.awq_s;
            if (arena && numel > 0) {
                if (p.awq_off < 0) return PGQ_ERR_PARAM;
                d.awq_out = reinterpret_cast<uint16_t*>(arena + p.awq_off);
            }
        }
    }
    return PGQ_OK;
}

// ---- the allocation-free export's scratch ------------------------------------------------------
// pgq_export_model_noalloc keeps its descriptor table (and the whole-tensor select state) in this
// file-scope array instead of a caller workspace.  Each GPU holds its own copy until the process
// ends; in host code `scratch` only names the symbol, so its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that address is used.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;         // per device: the address of that device's `scratch`

pgq_status scratch_for_current_device(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_failed(e);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_failed(e);
        if (!p) return PGQ_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PGQ_OK;
}

// Descriptors of an export call (shared by both export entry points).
pgq_status export_descs(const pgq_tensor_in* t, int32_t n, const pgq_tensor_plan* plan, void* arena,
                        float* const* dq_out, std::vector<Desc>& descs)
{
    if (!t || !plan) return PGQ_ERR_NULL;
    if (!arena) return PGQ_ERR_NULL;
    if (!aligned(arena, 256)) return PGQ_ERR_ALIGN;
    descs.resize((size_t)n);
    for (int32_t i = 0; i < n; ++i) {
        pgq_status st = check_tensor_in(t[i]);
        if (st != PGQ_OK) return st;
        st = check_plan_entry(plan[i]);
        if (st != PGQ_OK) return st;
        st = export_desc(t[i], plan[i], static_cast<uint8_t*>(arena), descs[i]);
        if (st != PGQ_OK) return st;
        if (dq_out && dq_out[i]) {
            if (!aligned(dq_out[i], 4)) return PGQ_ERR_ALIGN;
            descs[i].dq = dq_out[i];
        }
        set_vec_flag(descs[i]);
        set_grouping(descs[i], MODE_EXPORT);
    }
    return PGQ_OK;
}

}  // namespace

// The checks and launch of both GEMM entry points; esz = bytes of a Y element (4 or 2).
static pgq_status qgemm(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* codes, int64_t ldc,
                        const uint16_t* scales, int64_t N, void* y, int64_t ldy, int esz, void* stream)
{
    if (M < 0 || N < 0 || K < 0 || ldx < K || ldc < K || ldy < N) return PGQ_ERR_SHAPE;
    if (M > (int64_t)65535 * 128 || N > ((int64_t)1 << 31) || K > ((int64_t)1 << 31)) return PGQ_ERR_SHAPE;
    if (M == 0 || N == 0) return PGQ_OK;
    if (!y || (K > 0 && (!x || !codes || !scales))) return PGQ_ERR_NULL;
    if ((x && !aligned(x, 2)) || (scales && !aligned(scales, 2)) || !aligned(y, esz)) return PGQ_ERR_ALIGN;
    uint32_t f = 0;
    if (x && ldx % 8 == 0 && aligned(x, 16)) f |= 1u;
    if (codes && ldc % 16 == 0 && aligned(codes, 16)) f |= 2u;
    if (ldy % (16 / esz) == 0 && aligned(y, 16)) f |= 4u;
    if (const int e = launch_qgemm(x, M, K, ldx, codes, ldc, scales, N, y, ldy, esz == 2, f, stream))
        return hip_failed((hipError_t)e);
    if (const hipError_t e = hipGetLastError()) return hip_failed(e);
    return PGQ_OK;
}

extern "C" {

const char* pgq_version(void) { return "pgq 0.1 (gfx950)"; }

const char* pgq_last_error(void)
{
    return t_last_hip == hipSuccess ? "" : hipGetErrorString(t_last_hip);
}

pgq_status pgq_time_next_launch(void* start_event, void* stop_event)
{
    set_timing_events(start_event, stop_event);
    return PGQ_OK;
}

const char* pgq_status_str(pgq_status s)
{
    switch (s) {
    case PGQ_OK: return "ok";
    case PGQ_ERR_NULL: return "required pointer is NULL";
    case PGQ_ERR_SHAPE: return "invalid shape (negative size, ld < cols, or too large)";
    case PGQ_ERR_DTYPE: return "unsupported element type";
    case PGQ_ERR_PARAM: return "invalid parameter (bits, percentile, mode, k or plan kind)";
    case PGQ_ERR_ALIGN: return "pointer not aligned to its element size";
    case PGQ_ERR_WORKSPACE: return "workspace missing or too small";
    case PGQ_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

pgq_status pgq_quantize_rows(const void* w, int32_t w_dtype, int64_t rows, int64_t cols, int64_t ld,
                             pgq_qparams qp, const float* awq_s, uint16_t* awq_mult,
                             int8_t* codes, uint16_t* scales, void* dq, int32_t dq_dtype,
                             uint32_t* dev_status, void* stream)
{
    if (!shape_ok(rows, cols, ld)) return PGQ_ERR_SHAPE;
    if (!weight_dtype_ok(w_dtype)) return PGQ_ERR_DTYPE;
    if (dq && dq_dtype != PGQ_F32 && dq_dtype != PGQ_BF16) return PGQ_ERR_DTYPE;
    if (!qparams_ok(qp)) return PGQ_ERR_PARAM;
    if (rows == 0) return PGQ_OK;
    if (cols == 0) return PGQ_ERR_SHAPE;
    if (!w || !scales) return PGQ_ERR_NULL;
    if (awq_mult && !awq_s) return PGQ_ERR_NULL;
    if (!aligned(w, esize(w_dtype)) || !aligned(scales, 2) || (dq && !aligned(dq, esize(dq_dtype))) ||
        (awq_s && !aligned(awq_s, 4)) || (awq_mult && !aligned(awq_mult, 2)))
        return PGQ_ERR_ALIGN;
    Desc d = blank_desc();
    d.w = w;
    d.codes = codes;
    d.scales = scales;
    d.dq = dq;
    d.awq_s = awq_s;
    d.awq_out = awq_mult;
    d.rows = rows;
    d.cols = cols;
    d.ld = ld;
    d.kind = qp.bits;
    d.Q = (1 << (qp.bits - 1)) - 1;
    d.rank_top = rank_top(cols, qp.pct_num, qp.pct_den);
    d.in_dtype = in_of(w_dtype);
    d.dq_dtype = dq_dtype == PGQ_F32 ? IN_F32 : IN_BF16;
    set_vec_flag(d);
    set_grouping(d, MODE_EXPORT);
    return run_single(MODE_EXPORT, d, dev_status, 0, 0, stream);
}

pgq_status pgq_fakequant_workspace(const pgq_fq_tensor* t, int32_t n, size_t* workspace_bytes)
{
    if (!workspace_bytes) return PGQ_ERR_NULL;
    if (n < 0) return PGQ_ERR_SHAPE;
    if (n > 0 && !t) return PGQ_ERR_NULL;
    uint64_t nt = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (!shape_ok(t[i].rows, t[i].cols, t[i].ld)) return PGQ_ERR_SHAPE;
        nt += max_tiles_for(t[i].rows, t[i].cols);
    }
    *workspace_bytes = table_bytes((size_t)n, nt);
    return PGQ_OK;
}

pgq_status pgq_fakequant_fwd_bwd(int32_t mode, const pgq_fq_tensor* t, int32_t n, pgq_qparams qp,
                                 void* workspace, size_t workspace_bytes, uint32_t flags,
                                 uint32_t* dev_status, void* stream)
{
    if (mode != PGQ_FQ_FWD && mode != PGQ_FQ_BWD && mode != PGQ_FQ_FWD_BWD) return PGQ_ERR_PARAM;
    if (!qparams_ok(qp)) return PGQ_ERR_PARAM;
    if (n < 0) return PGQ_ERR_SHAPE;
    if (n == 0) return PGQ_OK;
    if (!t) return PGQ_ERR_NULL;
    const bool fwd = mode & PGQ_FQ_FWD, bwd = mode & PGQ_FQ_BWD;
    std::vector<Desc> descs((size_t)n);
    for (int32_t i = 0; i < n; ++i) {
        const pgq_fq_tensor& x = t[i];
        if (!shape_ok(x.rows, x.cols, x.ld)) return PGQ_ERR_SHAPE;
        if (x.rows > 0 && x.cols == 0) return PGQ_ERR_SHAPE;
        Desc& d = descs[i];
        d = blank_desc();
        d.rows = x.rows;
        d.cols = x.cols;
        d.ld = x.ld;
        d.kind = qp.bits;
        d.Q = (1 << (qp.bits - 1)) - 1;
        d.rank_top = rank_top(x.cols, qp.pct_num, qp.pct_den);
        d.in_dtype = IN_BF16;
        d.dq_dtype = IN_BF16;
        if (x.rows == 0) continue;
        if (fwd) {
            if (!x.w || !x.dq || !x.scales) return PGQ_ERR_NULL;
            d.w = x.w;
            d.dq = x.dq;
            d.scales = x.scales;
            d.codes = x.codes;
            d.mask = x.mask;
        } else {
            if (!x.mask) return PGQ_ERR_NULL;
            d.mask = x.mask;
            d.ld = x.cols;
        }
        if (bwd) {
            if (!x.grad || !x.grad_out) return PGQ_ERR_NULL;
            d.grad = x.grad;
            d.grad_out = x.grad_out;
        }
        if ((d.w && !aligned(d.w, 2)) || (d.dq && !aligned(d.dq, 2)) || (d.scales && !aligned(d.scales, 2)) ||
            (d.grad && !aligned(d.grad, 2)) || (d.grad_out && !aligned(d.grad_out, 2)))
            return PGQ_ERR_ALIGN;
        if (fwd) {
            set_vec_flag(d);
        } else {
            const bool ok = d.cols % 8 == 0 && aligned(d.grad, 16) && aligned(d.grad_out, 16);
            d.flags = ok ? DF_VEC : 0u;
        }
        set_grouping(d, fwd ? MODE_FQ : MODE_FQ_BWD);
    }
    const int kmode = fwd ? MODE_FQ : MODE_FQ_BWD;
    if (n == 1 && !workspace) return run_single(kmode, descs[0], dev_status, 0, mode, stream);
    return run_grouped(kmode, descs, workspace, workspace_bytes, flags, dev_status, 0, mode, stream);
}

pgq_status pgq_export_plan(const pgq_tensor_in* t, int32_t n, const pgq_policy* pol,
                           pgq_tensor_plan* plan, size_t* arena_bytes, size_t* workspace_bytes)
{
    if (n < 0) return PGQ_ERR_SHAPE;
    if (!pol || !arena_bytes || !workspace_bytes || (n > 0 && (!t || !plan))) return PGQ_ERR_NULL;
    if (pol->n_patterns < 0 || (pol->n_patterns > 0 && !pol->int8_patterns)) return PGQ_ERR_PARAM;
    if (!qparams_ok(pol->q_default) || !qparams_ok(pol->q_sensitive) || pol->passthrough_below < 0)
        return PGQ_ERR_PARAM;
    if (pol->per_tensor != 0 && pol->per_tensor != 1) return PGQ_ERR_PARAM;
    if (pol->pack6 != 0 && pol->pack6 != 1) return PGQ_ERR_PARAM;
    int64_t off = 0;
    uint64_t nt = 0, cand = 0;
    for (int32_t i = 0; i < n; ++i) {
        const pgq_tensor_in& x = t[i];
        nt += max_tiles_for(x.rows, x.cols);
        pgq_status st = check_tensor_in(x);
        if (st != PGQ_OK) return st;
        pgq_tensor_plan& p = plan[i];
        memset(&p, 0, sizeof(p));
        p.codes_off = p.scales_off = p.f16_off = p.awq_off = -1;
        const int64_t numel = x.rows * x.cols;
        if (numel < pol->passthrough_below) {
            p.kind = PGQ_KIND_F16;
            p.f16_off = off;
            off = align_up(off + numel * 2, 256);
        } else {
            const bool sens = name_matches(x.name, pol);
            p.qp = sens ? pol->q_sensitive : pol->q_default;
            p.kind = p.qp.bits;
            p.has_awq = (!sens && x.awq_s) ? 1 : 0;
            p.per_tensor = pol->per_tensor ? 1 : 0;
            if (p.per_tensor && p.has_awq) return PGQ_ERR_PARAM;
            if (p.per_tensor && numel >= (int64_t(1) << 32)) return PGQ_ERR_SHAPE;
            if (p.per_tensor) cand += cand_words_bound(x.rows, x.cols, x.dtype, rank_top(numel, p.qp.pct_num, p.qp.pct_den));
            p.packed = (pol->pack6 && p.kind == 6) ? 1 : 0;
            p.codes_off = off;
            off = align_up(off + (p.packed ? x.rows * (3 * ((x.cols + 3) / 4)) : numel), 256);
            p.scales_off = off;
            off = align_up(off + (p.per_tensor ? 1 : x.rows) * 2, 256);
            if (p.has_awq) {
                p.awq_off = off;
                off = align_up(off + x.cols * 2, 256);
            }
        }
    }
    *arena_bytes = (size_t)std::max<int64_t>(off, 256);
    *workspace_bytes = table_bytes((size_t)n, nt, cand);
    return PGQ_OK;
}

pgq_status pgq_export_model(const pgq_tensor_in* t, int32_t n, const pgq_tensor_plan* plan,
                            void* arena, float* const* dq_out, void* workspace, size_t workspace_bytes,
                            uint32_t flags, uint32_t* dev_status, void* stream)
{
    if (n < 0) return PGQ_ERR_SHAPE;
    if (n == 0) return PGQ_OK;
    std::vector<Desc> descs;
    const pgq_status st = export_descs(t, n, plan, arena, dq_out, descs);
    if (st != PGQ_OK) return st;
    return run_grouped(MODE_EXPORT, descs, workspace, workspace_bytes, flags, dev_status, 0, 0, stream);
}

pgq_status pgq_export_model_noalloc(const pgq_tensor_in* t, int32_t n, const pgq_tensor_plan* plan, void* arena,
                                    float* const* dq_out, uint32_t flags, uint32_t* dev_status, void* stream)
{
    if (n < 0) return PGQ_ERR_SHAPE;
    if (n == 0) return PGQ_OK;
    std::vector<Desc> descs;
    pgq_status st = export_descs(t, n, plan, arena, dq_out, descs);
    if (st != PGQ_OK) return st;
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != PGQ_OK) return st;
    // a table larger than the array is refused (PGQ_ERR_WORKSPACE) before anything is enqueued
    return run_grouped(MODE_EXPORT, descs, ws, kScratchBytes, flags, dev_status, 0, 0, stream);
}

pgq_status pgq_sqwa_accumulate(const pgq_tensor_in* snap, int32_t n, const pgq_tensor_plan* plan,
                               float* const* mean, int32_t k, void* workspace, size_t workspace_bytes,
                               uint32_t flags, uint32_t* dev_status, void* stream)
{
    if (n < 0) return PGQ_ERR_SHAPE;
    if (k < 1 || k > (1 << 24)) return PGQ_ERR_PARAM;     // k must be exact in binary32
    if (n == 0) return PGQ_OK;
    if (!snap || !plan || !mean) return PGQ_ERR_NULL;
    std::vector<Desc> descs((size_t)n);
    for (int32_t i = 0; i < n; ++i) {
        pgq_status st = check_tensor_in(snap[i]);
        if (st != PGQ_OK) return st;
        st = check_plan_entry(plan[i]);
        if (st != PGQ_OK) return st;
        if (plan[i].kind != PGQ_KIND_F16 && plan[i].per_tensor) return PGQ_ERR_PARAM;
        st = export_desc(snap[i], plan[i], nullptr, descs[i]);
        if (st != PGQ_OK) return st;
        if (snap[i].rows > 0 && snap[i].cols > 0) {
            if (!mean[i]) return PGQ_ERR_NULL;
            if (!aligned(mean[i], 4)) return PGQ_ERR_ALIGN;
        }
        descs[i].mean = mean[i];
        set_vec_flag(descs[i]);
        set_grouping(descs[i], MODE_SQWA);
    }
    return run_grouped(MODE_SQWA, descs, workspace, workspace_bytes, flags, dev_status, k, 0, stream);
}

pgq_status pgq_qgemm_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* codes, int64_t ldc,
                          const uint16_t* scales, int64_t N, float* y, int64_t ldy, void* stream)
{
    return qgemm(x, M, K, ldx, codes, ldc, scales, N, y, ldy, 4, stream);
}

pgq_status pgq_qgemm_bf16_ybf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* codes,
                                int64_t ldc, const uint16_t* scales, int64_t N, uint16_t* y, int64_t ldy, void* stream)
{
    return qgemm(x, M, K, ldx, codes, ldc, scales, N, y, ldy, 2, stream);
}

pgq_status pgq_dequant_codes(const void* codes, int32_t packed, int64_t rows, int64_t cols, const uint16_t* scales,
                             int32_t per_tensor, const uint16_t* awq_mult, float* out, uint32_t* dev_status,
                             void* stream)
{
    (void)dev_status;
    if (rows < 0 || cols < 0 || rows >= (int64_t(1) << 40) || cols > (int64_t(1) << 29) - 64) return PGQ_ERR_SHAPE;
    if ((packed != 0 && packed != 1) || (per_tensor != 0 && per_tensor != 1)) return PGQ_ERR_PARAM;
    if (rows == 0 || cols == 0) return PGQ_OK;
    if (!codes || !scales || !out) return PGQ_ERR_NULL;
    if (!aligned(scales, 2) || (awq_mult && !aligned(awq_mult, 2)) || !aligned(out, 4)) return PGQ_ERR_ALIGN;
    if (const int e = launch_decode(codes, packed, rows, cols, scales, per_tensor, awq_mult, out, stream))
        return hip_failed((hipError_t)e);
    if (const hipError_t e = hipGetLastError()) return hip_failed(e);
    return PGQ_OK;
}

pgq_status pgq_dequant_model(const pgq_tensor_in* t, int32_t n, const pgq_tensor_plan* plan, const void* arena,
                             float* const* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                             uint32_t* dev_status, void* stream)
{
    if (n < 0) return PGQ_ERR_SHAPE;
    if (n == 0) return PGQ_OK;
    if (!t || !plan || !arena || !out) return PGQ_ERR_NULL;
    if (!aligned(arena, 256)) return PGQ_ERR_ALIGN;
    const uint8_t* a = static_cast<const uint8_t*>(arena);
    std::vector<Desc> descs;
    descs.reserve((size_t)n);
    for (int32_t i = 0; i < n; ++i) {
        if (!shape_ok(t[i].rows, t[i].cols, t[i].ld)) return PGQ_ERR_SHAPE;
        const pgq_tensor_plan& p = plan[i];
        const pgq_status st = check_plan_entry(p);
        if (st != PGQ_OK) return st;
        if (!out[i] || t[i].rows == 0 || t[i].cols == 0) continue;
        if (!aligned(out[i], 4)) return PGQ_ERR_ALIGN;
        Desc d = blank_desc();
        d.rows = t[i].rows;
        d.cols = t[i].cols;
        d.ld = t[i].cols;
        d.dq = out[i];
        if (p.kind == PGQ_KIND_F16) {
            if (p.f16_off < 0) return PGQ_ERR_PARAM;
            d.kind = KIND_F16;
            d.f16_out = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(a + p.f16_off));
        } else {
            if (p.codes_off < 0 || p.scales_off < 0 || (p.has_awq && p.awq_off < 0)) return PGQ_ERR_PARAM;
            d.kind = p.kind;
            d.codes = reinterpret_cast<int8_t*>(const_cast<uint8_t*>(a + p.codes_off));
            d.scales = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(a + p.scales_off));
            if (p.has_awq) d.awq_out = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(a + p.awq_off));
            if (p.packed) d.flags |= DF_PACK6;
            if (p.per_tensor) d.flags |= DF_TENSOR;
        }
        // vector path: whole groups of four, 16-byte fp32 stores, 4-byte int8 code loads
        if (d.cols % 4 == 0 && aligned(out[i], 16)) d.flags |= DF_VEC;
        set_grouping(d, MODE_DECODE);
        descs.push_back(d);
    }
    if (descs.empty()) return PGQ_OK;
    return run_grouped(MODE_DECODE, descs, workspace, workspace_bytes, flags, dev_status, 0, 0, stream);
}

pgq_status pgq_average_workspace(const pgq_tensor_in* t, int32_t n, size_t* workspace_bytes)
{
    if (!workspace_bytes) return PGQ_ERR_NULL;
    if (n < 0) return PGQ_ERR_SHAPE;
    if (n > 0 && !t) return PGQ_ERR_NULL;
    uint64_t nt = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (!shape_ok(t[i].rows, t[i].cols, t[i].ld)) return PGQ_ERR_SHAPE;
        nt += max_tiles_for(t[i].rows, t[i].cols);
    }
    *workspace_bytes = table_bytes((size_t)n, nt);
    return PGQ_OK;
}

pgq_status pgq_ema_update(const pgq_tensor_in* w, int32_t n, float* const* ema, float decay, int32_t init,
                          void* workspace, size_t workspace_bytes, uint32_t flags, uint32_t* dev_status,
                          void* stream)
{
    if (n < 0) return PGQ_ERR_SHAPE;
    if (!(decay >= 0.0f && decay <= 1.0f)) return PGQ_ERR_PARAM;
    if (n == 0) return PGQ_OK;
    if (!w || !ema) return PGQ_ERR_NULL;
    std::vector<Desc> descs;
    const pgq_status st = average_descs(w, n, ema, MODE_EMA, descs);
    if (st != PGQ_OK) return st;
    const float c = 1.0f - decay;              // binary32, formed once
    return run_grouped(MODE_EMA, descs, workspace, workspace_bytes, flags, dev_status, 0, 0, stream,
                       init ? 1 : 0, decay, c);
}

pgq_status pgq_swa_accumulate(const pgq_tensor_in* w, int32_t n, float* const* mean, int32_t k, void* workspace,
                              size_t workspace_bytes, uint32_t flags, uint32_t* dev_status, void* stream)
{
    if (n < 0) return PGQ_ERR_SHAPE;
    if (k < 1 || k > (1 << 24)) return PGQ_ERR_PARAM;     // k must be exact in binary32
    if (n == 0) return PGQ_OK;
    if (!w || !mean) return PGQ_ERR_NULL;
    std::vector<Desc> descs;
    const pgq_status st = average_descs(w, n, mean, MODE_SWA, descs);
    if (st != PGQ_OK) return st;
    return run_grouped(MODE_SWA, descs, workspace, workspace_bytes, flags, dev_status, k, 0, stream);
}

}  // extern "C"
