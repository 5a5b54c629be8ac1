// pgq_desc.h -- descriptors shared by the host layer and the gfx950 kernels of libpgq.
//
// A launch processes "tiles": each tile is tile_rows consecutive rows of one tensor (four
// wavefronts, each taking rgroup rows at a time).  Grouped calls put a descriptor table
// into the caller's workspace: header, one Desc per tensor, tile_start[n + 1] (the first
// tile of each tensor, a prefix sum) and tile_desc[n_tiles] (the tensor of each tile).
// Single-matrix calls pass one Desc by value in the kernel arguments.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pgq {

constexpr int kWaves = 4;                 // wavefronts per workgroup
constexpr int kBlock = 64 * kWaves;       // threads per workgroup
constexpr uint64_t kTableMagic = 0x5047515441424c31ull;   // "PGQTABL1"

enum Mode : int32_t {
    MODE_EXPORT = 0, MODE_SQWA = 1, MODE_FQ = 2, MODE_FQ_BWD = 3, MODE_EMA = 4, MODE_SWA = 5,
    MODE_TSEL = 6,    // one pass of the whole-tensor clip select (per-tensor scales)
    MODE_EXPORT6 = 7, // export whose int6 codes are stored 4 per 3 bytes (a separate build of the
                      // export kernels, so the plain export keeps its register budget)
    MODE_DECODE = 8,  // stored artifact (codes / packed codes / fp16) back to fp32
    MODE_TCAND = 9    // whole-tensor clip, one read: every workgroup emits its candidate keys
};
constexpr int kModes = 10;
template <int M>
constexpr bool is_export = M == MODE_EXPORT || M == MODE_EXPORT6;
enum : int32_t { IN_F32 = 0, IN_BF16 = 1, IN_F16 = 2 };
enum : int32_t { KIND_F16 = 16 };
enum : uint32_t {
    DF_VEC = 1u,          // 16-byte vector path allowed for this tensor
    DF_TENSOR = 2u,       // one scale for the whole tensor, clip from its TState
    DF_PACK6 = 4u,        // codes stored 4 per 3 bytes (6-bit fields), 3 * ceil(cols / 4) per row
    DF_CAND = 8u,         // DF_TENSOR clip found from candidate keys (MODE_TCAND) instead of the
                          // radix passes (MODE_TSEL)
    DF_FLAT = 16u         // bf16 rows of cols / 8 >= 64 chunks, read rgroup rows at a time as one run
                          // of nch wave-wide loads (dense, absmax, per row)
};

// Features a launch needs; each kernel instantiation covers a fixed set of them, and the
// host launches the leanest one that covers what its tensors need (fewer paths compiled
// in means fewer registers and higher occupancy).
enum : uint32_t {
    F_F32 = 1u,       // fp32 inputs
    F_BF16 = 2u,      // bf16 inputs
    F_PASS = 4u,      // fp16 passthrough tensors
    F_AWQ = 8u,       // AWQ column multipliers
    F_SEL = 16u,      // clip below the row maximum (percentile select)
    F_SCALAR = 32u,   // unaligned tensors (element-wise path)
    F_LONG = 64u,     // rows longer than the register tile
    F_F16 = 128u,     // fp16 inputs
    F_ALL = 255u
};

// State of one tensor's whole-tensor clip select, in the caller's workspace.
// Candidate select (DF_CAND, one read of the tensor): every workgroup of the MODE_TCAND launch
// stores the keys of its rows that can still be the clip in its own slots of the tensor's
// candidate array (Desc::cand: ccap keys per tile, then one count per tile); the pick ranks them.
// Radix select: pass p adds every workgroup's LDS histogram of key digit p (bits 30..23,
// 22..15, 14..7, 6..0 of |x|, among the keys matching the digits already chosen) into hist[p];
// the digits chosen so far are re-derived from hist[0 .. p-1] by whoever needs them.
// The final pick stores the selected key and zeroes hist / kmax, so consecutive calls need no
// reset.
struct alignas(64) TState {
    uint32_t hist[4][256];
    uint32_t kmax;        // absmax select: running maximum key
    uint32_t key;         // the selected |x| bit pattern, read by the quantize pass
    uint32_t pad[14];
};

struct alignas(16) Desc {
    const void* w;            // input rows (fp32, bf16 or fp16), row stride ld elements
    int8_t* codes;            // rows x cols, dense
    uint16_t* scales;         // rows fp16
    void* dq;                 // rows x cols dense: fp32 or bf16 (dq_dtype)
    const float* awq_s;       // cols activation scales (AWQ) or null
    uint16_t* awq_out;        // cols fp16 multipliers a_j or null
    uint16_t* f16_out;        // passthrough: rows x cols fp16, dense
    float* mean;              // SQWA / SWA running mean or EMA state, rows x cols dense
    const uint16_t* grad;     // STE backward input (bf16, dense)
    uint16_t* grad_out;       // STE backward output (bf16, dense)
    uint8_t* mask;            // STE mask bits, rows x ceil(cols/8)
    TState* tstate;           // DF_TENSOR: the tensor's select state (workspace)
    int64_t rows, cols, ld;
    int64_t rank_top;         // the clip is the rank_top-th largest |x| of the row (1 = max)
    int32_t kind;             // code bits, or KIND_F16
    int32_t Q;                // 2^(bits-1) - 1
    int32_t in_dtype;         // IN_F32 / IN_BF16 / IN_F16
    int32_t dq_dtype;         // IN_F32 / IN_BF16
    uint32_t flags;           // DF_*
    int32_t rgroup;           // rows a wave processes together (1, 2, 4 or 8)
    int32_t tile_rows;        // rows per tile: kWaves * rgroup * groups per wave
    int32_t nch;              // vector path: ceil(chunks / 64) per row, 0 when the row streams
    uint32_t* cand;           // DF_CAND: candidate keys (workspace): ccap per tile, then a count per tile
    int32_t crows;            // DF_CAND: rows per candidate tile (kWaves * rows per wave)
    int32_t ccap;             // DF_CAND: most keys a candidate tile stores (a multiple of 4)
};

struct alignas(64) TableHeader {
    uint64_t magic;
    uint64_t checksum;
    uint32_t n_desc;
    uint32_t n_tiles;
    uint32_t pad[10];
};

struct KArgs {
    const TableHeader* hdr;       // grouped launches only (passed as separate kernel arguments)
    const Desc* table;
    const uint32_t* tile_start;   // n_desc + 1 entries
    const uint32_t* tile_desc;    // n_tiles entries
    uint64_t checksum;
    uint32_t* status;
    uint32_t n_tiles;
    int32_t sqwa_k;               // SQWA / SWA: 1-based snapshot index
    int32_t fq_mode;              // PGQ_FQ_* for MODE_FQ
    int32_t avg_init;             // EMA: nonzero starts the average at the weights
    float avg_d;                  // EMA: decay d
    float avg_c;                  // EMA: fl32(1 - d)
    int32_t tsel_pass;            // MODE_TSEL: 0 .. 3 (digits of bits 30..23, 22..15, 14..7, 6..0)
    int32_t tsel_group;           // MODE_TSEL: export tiles per select tile
    int32_t reserved;
};

// Host-side launcher implemented next to the kernels.
// need: the F_* features of the launch.  variant_of() names the instantiation used (its
// feature set); launch() takes the same `need`.
// single: the descriptor of a single-matrix launch, or null for a grouped (table) launch.
uint32_t variant_of(int mode, uint32_t need);
int launch(int mode, uint32_t need, const KArgs& ka, const Desc* single, uint32_t grid, void* stream);
// The next launch on this host thread records these hipEvent_t at kernel start / end (either
// may be null); take_timing_events() hands back and clears a pending pair.
void set_timing_events(void* start, void* stop);
void take_timing_events(void** start, void** stop);
// Any kernel with a 3-D grid, taking a pending timing-event pair like the others.
hipError_t launch_plain(const void* fn, dim3 grid, dim3 block, void** args, void* stream);
// The fused-dequant GEMM (pgq_gemm.hip), Y fp32 or (ybf16) bf16; flags: bit 0 X rows 16-byte
// loadable, bit 1 code rows, bit 2 Y rows 16-byte aligned.
int launch_qgemm(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const int8_t* codes, int64_t ldc,
                 const uint16_t* scales, int64_t N, void* y, int64_t ldy, bool ybf16, uint32_t flags, void* stream);
// Decode of stored codes to fp32 (rows > 0, cols > 0).
int launch_decode(const void* codes, int32_t packed, int64_t rows, int64_t cols, const uint16_t* scales,
                  int32_t per_tensor, const uint16_t* awq, float* out, void* stream);
// The final pick of the whole-tensor selects: one workgroup per descriptor.
int launch_tensor_pick(const KArgs& ka, uint32_t n_desc, void* stream);

// Kernel instantiations for a variant v = variant_of(mode, need), grouped by mode into translation
// units of their own (pgq_k_*.hip) so that they compile in parallel; null when none exists.
// Export-like modes: kernels_<mode> holds the lean streaming variants, kernels_<mode>_sel the
// percentile-select variant, kernels_<mode>_all_* the variant with every feature.
#define PGQ_EXPORT_LIKE_PARTS(m)                                \
    const void* kernels_##m(uint32_t v, bool table);             \
    const void* kernels_##m##_sel(bool table);                   \
    const void* kernels_##m##_all_table();                       \
    const void* kernels_##m##_all_single();
PGQ_EXPORT_LIKE_PARTS(export)
PGQ_EXPORT_LIKE_PARTS(export6)
PGQ_EXPORT_LIKE_PARTS(sqwa)
#undef PGQ_EXPORT_LIKE_PARTS
const void* kernels_fq(int mode, uint32_t v, bool table);
const void* kernels_avg(int mode, uint32_t v, bool table);

// Register tile: a row of up to 64 * chunks * elements stays in VGPRs; longer rows stream.
constexpr int64_t kRegCols_F32 = 64 * 8 * 4;     // 2048
constexpr int64_t kRegCols_BF16 = 64 * 4 * 8;    // 2048
constexpr int64_t kRegCols_Scalar = 64 * 16;     // 1024

}  // namespace pgq
