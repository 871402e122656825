// C ABI of normhip: argument validation, launch planning, per-kernel timing.
// Every entry point validates all arguments before the first HIP call that
// could launch work, so a failing call writes nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "nh_bn.hpp"
#include "nh_internal.hpp"
#include "nh_rows.hpp"
#include "normhip.h"

using namespace nh;

namespace {

thread_local std::string g_last_error;

nh_status fail(nh_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
nh_status fail(nh_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

nh_status ok()
{
    g_last_error.clear();
    return NH_OK;
}

nh_status hip_fail(hipError_t e, const char *what)
{
    return fail(NH_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxElems = (int64_t)1 << 31;  // exclusive bound: 32-bit device indexing

bool valid_dtype(int t) { return t == NH_F32 || t == NH_BF16; }
size_t dtype_bytes(int t) { return t == NH_F32 ? 4 : 2; }
bool aligned(const void *p, size_t a) { return p == nullptr || ((uintptr_t)p % a) == 0; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- device properties, cached per device -----------------------------------
struct DeviceInfo {
    bool valid = false;
    int cus = 0;
    int threads_per_cu = 0;
    size_t lds_per_block = 0;
};

std::mutex g_dev_mu;
DeviceInfo g_dev[64];
std::map<int64_t, int> g_rows_occupancy;  // (device, variant) -> blocks per CU

nh_status device_info(DeviceInfo *out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(NH_ERR_HIP, "device id %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (!g_dev[dev].valid) {
        hipDeviceProp_t p;
        e = hipGetDeviceProperties(&p, dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
        g_dev[dev].cus = p.multiProcessorCount;
        g_dev[dev].threads_per_cu = p.maxThreadsPerMultiProcessor;
        g_dev[dev].lds_per_block = p.sharedMemPerBlock;
        g_dev[dev].valid = true;
    }
    *out = g_dev[dev];
    return NH_OK;
}

// ---- plan overrides ------------------------------------------------------------
std::atomic<int64_t> g_override_bn_grid_y{0};
std::atomic<int64_t> g_override_bn_ew_grid_y{0};
std::atomic<int64_t> g_override_rows_blocks{0};
std::atomic<int64_t> g_override_bn_finalize_kernels{0};
std::atomic<int64_t> g_override_rows_depth{0};
std::atomic<int64_t> g_override_colsum_cols{0};
std::atomic<int64_t> g_override_rows_teams{0};
std::atomic<int64_t> g_override_bn_channel{0};
std::atomic<int64_t> g_override_bn_channel_threads{0};
std::atomic<int64_t> g_override_rows_narrow{0};
std::atomic<int64_t> g_override_bn_block_order{0};
std::atomic<int64_t> g_override_bn_unit_order{0};

// ---- BatchNorm planning ----------------------------------------------------------
// Resident 256-thread block slots of the device: CUs * (threads per CU / 256),
// the rule of Aether-ML PR #18's "Reduction grid" section.
int64_t bn_slots(const DeviceInfo &d)
{
    int64_t per_cu = d.threads_per_cu / kBnThreads;
    if (per_cu < 1) per_cu = 1;
    return (int64_t)d.cus * per_cu;
}

// Unit assignment of the split BatchNorm passes (bn_range): interleaved
// sweeps unless the "bn_unit_order" override asks for contiguous ranges (1)
// (2 is the automatic choice).  Interleaved only where every block of the
// channel gets at least one whole sweep; with fewer units per channel some
// blocks would sit idle.  bn_auto_grid_y sizes the grid for it.
bool bn_interleave_wanted() { return g_override_bn_unit_order.load() != 1; }
int bn_interleave(int64_t units, int64_t grid_y)
{
    return bn_interleave_wanted() && units >= grid_y * kBnMinUnits ? 1 : 0;
}

// Blocks per channel of the reduction passes (stats, grad_sums); the
// workspace holds this many partial slots.
int64_t bn_grid_y_for(int64_t units, int64_t C, const DeviceInfo &d)
{
    const int64_t ov = g_override_bn_grid_y.load();
    if (ov > 0) return ov < units ? ov : units;
    return bn_auto_grid_y(units, C, bn_slots(d), bn_interleave_wanted());
}

// Blocks per channel of the elementwise passes (apply, dx, inference): the
// reductions' split unless a tuning override sets its own.
int64_t bn_ew_grid_y_for(int64_t units, int64_t C, const DeviceInfo &d)
{
    const int64_t ov = g_override_bn_ew_grid_y.load();
    if (ov > 0) return ov < units ? ov : units;
    return bn_grid_y_for(units, C, d);
}

// One block per channel (the fused kernels) for channels of at most
// kBnChannelMaxUnits units, or of at most twice that when the channels alone
// fill a quarter of the resident block slots; unless a grid or finalize
// override asks for the split path.  The "bn_channel" override forces it off
// (1) or on (2).  Measured on MI355X, fwd+bwd per step:
//   (3,37,41,40) fp32, 1230 units:   15.2 -> 10.9 us
//   (16,128,16,16) bf16, 512 units:  15.6 -> 9.7 us
//   (64,512,7,7) fp32, 3136 units:   22.8 -> 18.1 us
//   (64,2048,7,7) bf16, 3136 units:  52.6 -> 47.8 us
//   (256,64,8,8) fp32, 4096 units, 64 channels: 16.2 -> 17.9 us (split kept)
//   (64,256,28,28) bf16, 6272 units: 42.5 -> 53.5 us (split kept)
int bn_channel_fused(int64_t units, int64_t C, int64_t slots)
{
    const int64_t ov = g_override_bn_channel.load();
    if (ov == 1) return 0;
    if (ov == 2) return 1;
    if (g_override_bn_grid_y.load() > 0 || g_override_bn_ew_grid_y.load() > 0 ||
        g_override_bn_finalize_kernels.load() != 0)
        return 0;
    if (units <= kBnChannelMaxUnits) return 1;
    return units <= 2 * kBnChannelMaxUnits && 4 * C >= slots ? 1 : 0;
}

// Threads per block of the fused kernels: kBnChannelBigBlock (one sweep of
// a 4096-unit channel) when every such block stays resident and a 256-thread
// block would sweep more than once -- channels at most an eighth of the
// 256-thread slots with more than kBnMinUnits units, or at most a quarter
// with more than 2*kBnMinUnits -- else kBnThreads.  Measured on MI355X
// (fwd+bwd per step, 256 -> 1024 threads): (3,37,41,40) fp32 10.6 -> 9.7 us,
// (8,64,32,32) fp32 11.8 -> 10.7 us, (64,512,7,7) fp32 18.0 -> 15.5 us;
// (32,512,7,7) fp32 12.5 -> 13.1 us and (64,2048,7,7) bf16 48 -> 56 us keep
// 256.  The "bn_channel_threads" override forces either.
int bn_channel_threads(int64_t units, int64_t C, int64_t slots)
{
    const int64_t ov = g_override_bn_channel_threads.load();
    if (ov == kBnThreads || ov == kBnChannelBigBlock) return (int)ov;
    const bool big = (8 * C <= slots && units > kBnMinUnits) || (4 * C <= slots && units > 2 * kBnMinUnits);
    return big ? kBnChannelBigBlock : kBnThreads;
}

// Block numbering of the split BatchNorm passes (bn_block): channel-fastest
// unless the "bn_block_order" override asks for channel-major (1) or
// channel-fastest (2).  Measured on MI355X, cold per call, the same box,
// channel-major -> channel-fastest: (256,32,32,32) fp32 fwd+bwd 42.2 ->
// 40.5 us (all four passes faster), inference + ReLU at that shape 13.9 ->
// 13.0 us and at (64,256,56,56) bf16 39.1 -> 37.5 us; (64,256,56,56) bf16
// and (256,32,32,32) bf16 fwd+bwd within 0.5% either way.  A probe of the
// bare access pattern showed the same: reading the fp32 tensor by channel
// runs took 8.2 us in channel-major order, 7.4 us channel-fastest and 7.2 us
// as contiguous chunks.
int bn_chan_fast()
{
    const int64_t ov = g_override_bn_block_order.load();
    if (ov == 1) return 0;
    if (ov == 2) return 1;
    return 1;
}

// The finalize in the elementwise prologue reads a channel's partial slots
// (a row of grid_y floats) through buffer resources with 32-bit byte offsets
// yb*4: it runs there only while a row spans less than 2^31 bytes (always,
// short of a forced grid beyond 2^29 blocks per channel); else the finalize
// runs as its own kernel.
bool bn_fused_finalize_fits(int64_t grid_y) { return grid_y * 4 < ((int64_t)1 << 31); }

// Largest grid_y any dtype/alignment can take for this shape (scalar units).
int64_t bn_grid_y_max(int64_t M, int64_t C, const DeviceInfo &d) { return bn_grid_y_for(M, C, d); }

// Small planes take the row layout (bn_col_* kernels): planes of at most
// kBnColMaxPlaneBytes bytes, where the channel layout reads short runs
// scattered C*HW elements apart -- unless the channel layout would run one
// fused kernel per direction on vector units, which its two launches (against
// the row layout's three per direction) make faster.  Measured on MI355X,
// fwd+bwd per step, channel layout -> row layout:
//   (16384,2048,1,1) bf16  5774 -> 139 us     (4096,1024,1,1) fp32  521 -> 40.5 us
//   (65536,256,1,1) bf16   1428 -> 107 us     (64,2048,7,7) bf16    48.1 -> 34.3 us
//   but (256,512,4,4) fp32 17.3 -> 26.1 us and (128,256,8,8) bf16 14.3 -> 29.0 us
//   (fused, vector units: kept on the channel layout).
// `chan_vec` and `fused` are the channel layout's unit width and fused-kernel
// choice (fused = 0 for inference).  The "bn_layout" override forces the
// channel layout (1) or the row layout (2).
constexpr int64_t kBnColMaxPlaneBytes = 128;
std::atomic<int64_t> g_override_bn_layout{0};

bool bn_col_possible(int io, int64_t HW) { return HW * (io == NH_F32 ? 4 : 2) <= kBnColMaxPlaneBytes; }

bool bn_col_layout(int io, int64_t HW, int chan_vec, int fused)
{
    const int64_t ov = g_override_bn_layout.load();
    if (ov == 1) return false;
    if (ov == 2) return true;
    // overrides that shape the channel layout's plan ask for that layout
    if (g_override_bn_grid_y.load() > 0 || g_override_bn_ew_grid_y.load() > 0 ||
        g_override_bn_finalize_kernels.load() != 0 || g_override_bn_channel.load() == 2)
        return false;
    return bn_col_possible(io, HW) && (chan_vec == 1 || !fused);
}

// Workspace of the row layout for either dtype and unit width (the workspace
// query takes no dtype): partials[2, rb, C*HW].
size_t bn_col_ws_bytes(int64_t N, int64_t C, int64_t HW)
{
    const int64_t ov = g_override_bn_layout.load();
    if (ov == 1 || (ov != 2 && !bn_col_possible(NH_F32, HW) && !bn_col_possible(NH_BF16, HW))) return 0;
    return round_up((size_t)(2 * bn_col_chunks_max(N, C * HW) * C * HW) * sizeof(float), 256);
}

int bn_vec(int io, int64_t HW, const void *a, const void *b, const void *c);

// Row-layout plan: the unit width along the rows (bn_vec over the row length),
// the geometry; the one-block-per-channel kernels do not apply.
void bn_col_plan(BnCall &a, const void *p0, const void *p1, const void *p2)
{
    a.col = 1;
    a.channel_fused = 0;
    a.vec = bn_vec(a.io, (int64_t)a.C * a.HW, p0, p1, p2);
    a.colg = make_bn_col_geom(a.N, a.C, a.HW, a.vec);
}

size_t bn_ws_bytes(int64_t N, int64_t C, int64_t HW, const DeviceInfo &d)
{
    const int64_t M = N * HW;
    const size_t col = bn_col_ws_bytes(N, C, HW);
    // partials[C, 2, grid_y] + shifts K[C]
    const size_t chan = round_up((size_t)((2 * bn_grid_y_max(M, C, d) + 1) * C) * sizeof(float), 256);
    return chan > col ? chan : col;
}

nh_status bn_check_shape(int64_t N, int64_t C, int64_t HW)
{
    if (N < 0 || C < 0 || HW < 0) return fail(NH_ERR_SHAPE, "negative size (N=%lld C=%lld HW=%lld)",
                                              (long long)N, (long long)C, (long long)HW);
    if (N > 0 && C > 0 && HW > 0 && (N >= kMaxElems || C >= kMaxElems || HW >= kMaxElems ||
                                     N * C >= kMaxElems || N * C * HW >= kMaxElems))
        return fail(NH_ERR_SHAPE, "N*C*HW must be below 2^31");
    return NH_OK;
}

// Elements per BatchNorm unit: 16 bytes (4 fp32 / 8 bf16) when the plane
// length and the pointers allow it; for bf16, 8-byte units (4 elements) when
// only those fit (planes of 4k elements, e.g. 14x14); else single elements.
int bn_vec(int io, int64_t HW, const void *a, const void *b, const void *c)
{
    auto all_aligned = [&](size_t al) { return aligned(a, al) && aligned(b, al) && aligned(c, al); };
    if (io == NH_F32) return HW % 4 == 0 && all_aligned(16) ? 4 : 1;
    if (HW % 8 == 0 && all_aligned(16)) return 8;
    if (HW % 4 == 0 && all_aligned(8)) return 4;
    return 1;
}

// ---- rows planning ---------------------------------------------------------------
struct RowsPlan {
    int maxg = 0;   // 0 = generic path
    int vec = 1;
    int team = kTeam;
    int blocks = 0;
};

// Upper bound of the row kernels' block count G (the workspace holds G
// column-partial rows): kRowsMaxBlocksPerCu per CU, at most one per row.
int64_t rows_blocks_max(int64_t rows, const DeviceInfo &d)
{
    const int64_t ov = g_override_rows_blocks.load();
    int64_t g = ov > 0 ? ov : (int64_t)d.cus * kRowsMaxBlocksPerCu;
    if (g > kRowsMaxBlocks) g = kRowsMaxBlocks;
    if (g > rows) g = rows;
    return g;
}

// Partial rows the workspace holds: rows_blocks_max, or, for rows short
// enough for the lane-subgroup kernels (at most kGenNarrowMaxCols columns:
// short partial rows), up to kRowsMaxBlocks, since those kernels need many
// blocks to keep enough short rows in flight.
int64_t rows_partial_rows(int64_t rows, int64_t cols, const DeviceInfo &d)
{
    if (cols > kGenNarrowMaxCols) return rows_blocks_max(rows, d);
    const int64_t ov = g_override_rows_blocks.load();
    int64_t g = ov > 0 ? ov : kRowsMaxBlocks;
    if (g > kRowsMaxBlocks) g = kRowsMaxBlocks;
    if (g > rows) g = rows;
    return g;
}

// Workspace of a row backward: the partial rows [Q, G, cols] (G at most
// rows_partial_rows), then, for rows wider than kGenNarrowGroups that take
// the generic strip kernels, two fp32 sums per row segment
// (gen_coef_slots(rows) segments per row at most).
size_t rows_partials_bytes(int Q, int64_t rows, int64_t cols, const DeviceInfo &d)
{
    return round_up((size_t)(Q * rows_partial_rows(rows, cols, d) * cols) * sizeof(float), 256);
}

size_t rows_ws_bytes(int Q, int64_t rows, int64_t cols, const DeviceInfo &d)
{
    const size_t coef =
        cols > kGenNarrowGroups ? round_up((size_t)(rows * gen_coef_slots(rows)) * 2 * sizeof(float), 256) : 0;
    return rows_partials_bytes(Q, rows, cols, d) + coef;
}

// Kernel variant for a row width: vector groups per thread (maxg, 0 = the
// generic path) and the group width.  One 256-thread team per block.
RowsPlan rows_variant(int64_t cols, int vec, bool vec_ok, int max_elems = kRowsMaxRowElems)
{
    RowsPlan p;
    p.vec = vec;
    const int64_t groups = vec_ok && cols % vec == 0 ? cols / vec : -1;
    if (groups > 0) {
        const int64_t per_thread = ceil_div(groups, kTeam);
        int mg = 1;
        while (mg < per_thread) mg <<= 1;
        // A thread holds at most max_elems row elements in registers.
        if (mg <= 8 && mg * vec <= max_elems) {
            p.maxg = mg;
        } else if (ceil_div(groups, kWideTeam) * vec <= max_elems) {
            // Up to twice as wide: a 512-thread team at max_elems per thread.
            p.team = kWideTeam;
            p.maxg = max_elems / vec;
        }
    }
    if (p.maxg == 0) p.vec = 1;
    return p;
}

// Rows short enough for the narrow kernels (a lane subgroup per row): at
// most kGenNarrowGroups groups of `vec` elements.  With vector groups this
// also takes aligned rows the 256-thread team kernels would run with most of
// their threads idle and a block barrier per row -- measured on MI355X,
// RMSNorm backward 131072x128 bf16 203 us and 1048576x16 bf16 1604 us on
// the team kernel.  The "rows_narrow" override = 1 keeps aligned rows on the
// team kernels.
bool rows_narrow(int64_t cols, int vec)
{
    if (vec == 1) return cols <= kGenNarrowGroups;
    return g_override_rows_narrow.load() != 1 && cols / vec <= kGenNarrowGroups;
}

// Generic path (no vector variant fits): rows of at most kGenNarrowGroups
// columns take the narrow kernel with scalar accesses and a subgroup of ct
// lanes per row (ct = the power of two covering the row), each block's
// 256/ct row slots taking at least kGenNarrowRowsInFlight rows, up to
// rows_partial_rows blocks; wider rows take the coefficient
// and strip kernels with vec-element groups when the tensors allow it, in
// chunks of rows sized for about kGenTargetBlocks strip blocks, chunks of
// at least kGenMinChunkRows rows.  The block count (partial rows) never
// exceeds rows_partial_rows, which the workspace holds; the "rows_blocks"
// override forces it.
void rows_generic_plan(RowsCall &a, bool vec_ok, const DeviceInfo &d)
{
    const int64_t gmax = rows_partial_rows(a.rows, a.cols, d);
    const bool forced = g_override_rows_blocks.load() > 0;
    a.maxg = 0;
    a.team = kTeam;
    const int gvec = vec_ok && a.cols % a.vec == 0 ? a.vec : 1;
    const int64_t groups = a.cols / gvec;
    if (rows_narrow(a.cols, gvec)) {
        int ct = 1;
        while (ct < groups) ct <<= 1;
        const int64_t slots = kTeam / ct;
        int64_t g = forced ? gmax : ceil_div(a.rows, slots * kGenNarrowRowsInFlight);
        if (g > gmax) g = gmax;
        if (g < 1) g = 1;
        a.vec = gvec;
        a.gen_ct = ct;
        a.gen_rpc = 0;
        a.gen_coef_waves = 0;
        a.blocks = (int)g;
        return;
    }
    const int64_t strips = ceil_div(groups, kGenStripGroups);
    int64_t rb = forced ? gmax : std::min(ceil_div(kGenTargetBlocks, strips), ceil_div(a.rows, kGenMinChunkRows));
    if (rb > gmax) rb = gmax;
    if (rb < 1) rb = 1;
    const int64_t rpc = ceil_div(a.rows, rb);
    a.vec = gvec;
    a.gen_ct = 0;
    a.gen_rpc = (int)rpc;
    a.gen_coef_waves = groups >= kGenTeamCoefGroups ? kGenCoefTeamWaves : 1;
    int64_t segs = 1;
    if (a.gen_coef_waves > 1) {
        segs = std::min<int64_t>(gen_coef_slots(a.rows), groups / kGenCoefMinSegGroups);
        if (segs < 1) segs = 1;
    }
    a.gen_coef_segs = (int)segs;
    a.blocks = (int)ceil_div(a.rows, rpc);
}

// Forward generic path (no vector variant fits, or rows short enough for
// the narrow kernel, see rows_narrow): short rows take the narrow kernel (a
// subgroup of ct lanes per row, each row slot loading up to
// kGenNarrowRowsInFlight rows at once, at most 8 blocks per CU); wider rows
// a team per row with vec-element groups when the
// tensors allow it, 1024 threads when 256-thread teams would leave the device
// part empty and every thread still gets kGenFwdMinGroupsPerThread groups,
// one block per row up to a full device.
void rows_forward_generic_plan(FwdCall &a, bool vec_ok, const DeviceInfo &d)
{
    const int64_t full = (int64_t)d.cus * 8;  // resident 256-thread blocks
    a.maxg = 0;
    const int gvec = vec_ok && a.cols % a.vec == 0 ? a.vec : 1;
    const int64_t groups = a.cols / gvec;
    if (rows_narrow(a.cols, gvec)) {
        int ct = 1;
        while (ct < groups) ct <<= 1;
        int64_t g = ceil_div(a.rows, (int64_t)(kTeam / ct) * kGenNarrowRowsInFlight);
        if (g > full) g = full;
        if (g < 1) g = 1;
        a.vec = gvec;
        a.team = kTeam;
        a.gen_ct = ct;
        a.blocks = (int)g;
        return;
    }
    const bool big = a.rows < full && groups >= (int64_t)kGenFwdBigTeam * kGenFwdMinGroupsPerThread;
    a.vec = gvec;
    a.gen_ct = 0;
    a.team = big ? kGenFwdBigTeam : kTeam;
    const int64_t cap = full * kTeam / a.team;
    a.blocks = (int)(a.rows < cap ? a.rows : cap);
}

// Blocks: as many as fit on the device at once (occupancy of the chosen
// variant, at most rows_blocks_per_cu per CU), at most one per row.
// Measured on MI355X: a 256-thread team per row beats wider teams that
// synchronize more waves per row (512-thread teams only for rows a
// 256-thread team cannot hold).
void rows_grid(RowsPlan &p, int kind, int row_bytes, int64_t groups, int64_t rows, int occ,
               const DeviceInfo &d)
{
    const int per_cu = rows_blocks_per_cu(kind, row_bytes, groups);
    if (occ < 1) occ = 1;
    if (occ > per_cu) occ = per_cu;
    int64_t g = (int64_t)d.cus * occ;
    const int64_t ov = g_override_rows_blocks.load();
    if (ov > 0) g = ov;
    if (g > kRowsMaxBlocks) g = kRowsMaxBlocks;
    if (g > rows) g = rows;
    if (g < 1) g = 1;
    p.blocks = (int)g;
}

// ---- timing --------------------------------------------------------------------------
std::atomic<bool> g_timing{false};
std::mutex g_timing_mu;
struct TimingRec { int kid; hipEvent_t start, stop; };
std::vector<TimingRec> g_records;
std::vector<hipEvent_t> g_event_pool;
size_t g_pool_used = 0;

hipEvent_t pool_event()
{
    if (g_pool_used == g_event_pool.size()) {
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        g_event_pool.push_back(e);
    }
    return g_event_pool[g_pool_used++];
}

} // namespace

namespace nh {

bool timing_on() { return g_timing.load(std::memory_order_relaxed); }

void timing_events(int kid, hipEvent_t *start, hipEvent_t *stop)
{
    std::lock_guard<std::mutex> lk(g_timing_mu);
    hipEvent_t a = pool_event(), b = pool_event();
    if (!a || !b) { *start = *stop = nullptr; return; }
    g_records.push_back({kid, a, b});
    *start = a;
    *stop = b;
}

} // namespace nh

extern "C" {

const char *nh_status_string(int status)
{
    switch (status) {
    case NH_OK: return "NH_OK";
    case NH_ERR_NULL: return "NH_ERR_NULL";
    case NH_ERR_SHAPE: return "NH_ERR_SHAPE";
    case NH_ERR_DTYPE: return "NH_ERR_DTYPE";
    case NH_ERR_WORKSPACE: return "NH_ERR_WORKSPACE";
    case NH_ERR_HIP: return "NH_ERR_HIP";
    case NH_ERR_ARG: return "NH_ERR_ARG";
    default: return "NH_ERR_UNKNOWN";
    }
}

const char *nh_last_error(void) { return g_last_error.c_str(); }

const char *nh_kernel_name(int k)
{
    static const char *names[NH_K_COUNT] = {
        "bn_stats", "bn_fwd_finalize", "bn_apply", "bn_grad_sums", "bn_bwd_finalize", "bn_dx",
        "ln_rows", "ln_colsum", "rms_rows", "rms_colsum", "calib", "ln_fwd", "rms_fwd", "bn_infer",
        "bda_rows", "bda_colsum", "rows_coef", "bn_fwd_channel", "bn_bwd_channel"};
    return (k >= 0 && k < NH_K_COUNT) ? names[k] : "";
}

// ---- BatchNorm ---------------------------------------------------------------------
nh_status bn_forward_train_workspace(int64_t N, int64_t C, int64_t HW, size_t *ws_bytes)
{
    if (!ws_bytes) return fail(NH_ERR_NULL, "ws_bytes is NULL");
    nh_status st = bn_check_shape(N, C, HW);
    if (st != NH_OK) return st;
    if (N * C * HW == 0) { *ws_bytes = 0; return ok(); }
    DeviceInfo d;
    if ((st = device_info(&d)) != NH_OK) return st;
    *ws_bytes = bn_ws_bytes(N, C, HW, d);
    return ok();
}

nh_status bn_backward_workspace(int64_t N, int64_t C, int64_t HW, size_t *ws_bytes)
{
    return bn_forward_train_workspace(N, C, HW, ws_bytes);
}

static nh_status check_act(nh_act act, float slope)
{
    if (act != NH_ACT_NONE && act != NH_ACT_RELU && act != NH_ACT_LEAKY_RELU)
        return fail(NH_ERR_ARG, "act %d is not an nh_act value", (int)act);
    if (act == NH_ACT_LEAKY_RELU && !isfinite(slope)) return fail(NH_ERR_ARG, "slope must be finite");
    return NH_OK;
}

// The BatchNorm training forward, whole (stage 0) or one of its two stages.
// The launch plan every BatchNorm call shares: blocks per channel for the
// reduction and elementwise passes, block numbering, and the unit order.
static void bn_plan_grid(BnCall &a, nh_dtype io, int64_t N, int64_t C, int64_t HW, int vec, const DeviceInfo &d)
{
    a.io = io;
    a.N = (int)N;
    a.C = (int)C;
    a.HW = (int)HW;
    a.vec = vec;
    const int64_t units = N * (HW / vec);
    a.grid_y = (int)bn_grid_y_for(units, C, d);
    a.ew_grid_y = (int)bn_ew_grid_y_for(units, C, d);
    a.chan_fast = bn_chan_fast();
    a.ilv = bn_interleave(units, std::max(a.grid_y, a.ew_grid_y));
}

// The training calls' further choices: where the finalize runs, and whether
// one block per channel does the whole pass.
static void bn_plan_training(BnCall &a, const DeviceInfo &d)
{
    const int64_t units = (int64_t)a.N * (a.HW / a.vec);
    a.separate_finalize = g_override_bn_finalize_kernels.load() != 0 || !bn_fused_finalize_fits(a.grid_y);
    a.channel_fused = bn_channel_fused(units, a.C, bn_slots(d));
    a.channel_threads = bn_channel_threads(units, a.C, bn_slots(d));
}

static nh_status bn_forward_impl(int stage, const void *x, void *y, nh_dtype io, int64_t N, int64_t C,
                                 int64_t HW, const float *gamma, const float *beta, float *running_mean,
                                 float *running_var, float momentum, float eps, nh_act act, float slope,
                                 float *stats, void *ws, size_t ws_bytes, void *stream)
{
    if (!valid_dtype(io)) return fail(NH_ERR_DTYPE, "io dtype %d", (int)io);
    nh_status st = bn_check_shape(N, C, HW);
    if (st != NH_OK) return st;
    if (N * C * HW == 0) return ok();
    if (!x || !y || !stats) return fail(NH_ERR_NULL, "x, y and stats are required");
    const int64_t M = N * HW;
    if ((running_mean || running_var) && M < 2)
        return fail(NH_ERR_SHAPE, "running statistics need more than one element per channel");
    if (!(eps >= 0.f) || !isfinite(eps)) return fail(NH_ERR_ARG, "eps must be finite and >= 0");
    if (!isfinite(momentum)) return fail(NH_ERR_ARG, "momentum must be finite");
    if ((st = check_act(act, slope)) != NH_OK) return st;
    DeviceInfo d;
    if ((st = device_info(&d)) != NH_OK) return st;
    const size_t need = bn_ws_bytes(N, C, HW, d);
    if (!ws || ws_bytes < need || !aligned(ws, 16))
        return fail(NH_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned (got %zu)", need, ws_bytes);

    BnCall a{};
    bn_plan_grid(a, io, N, C, HW, bn_vec(io, HW, x, y, nullptr), d);
    a.x = x;
    a.out = y;
    a.gamma = gamma;
    a.beta = beta;
    a.running_mean = running_mean;
    a.running_var = running_var;
    a.momentum = momentum;
    a.eps = eps;
    a.act = act;
    a.slope = slope;
    a.stats = stats;
    a.partials = static_cast<float *>(ws);
    a.stage = stage;
    bn_plan_training(a, d);
    if (bn_col_layout(io, HW, a.vec, a.channel_fused)) bn_col_plan(a, x, y, nullptr);
    hipError_t e = bn_forward_launch(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "bn_forward_train launch");
    return ok();
}

nh_status bn_act_forward_train(const void *x, void *y, nh_dtype io, int64_t N, int64_t C, int64_t HW,
                               const float *gamma, const float *beta, float *running_mean,
                               float *running_var, float momentum, float eps, nh_act act, float slope,
                               float *stats, void *ws, size_t ws_bytes, void *stream)
{
    return bn_forward_impl(0, x, y, io, N, C, HW, gamma, beta, running_mean, running_var, momentum, eps, act,
                           slope, stats, ws, ws_bytes, stream);
}

// ---- the allocation-free training forward -----------------------------------
// bn_forward_train_noalloc keeps its workspace (the stats pass's partials and
// shifts) in this file-scope device array instead of a caller's buffer: one
// copy per GPU, held until the process ends.  Host code must not pass the
// array's name to a kernel (in host code it is a host-side stand-in, not a
// device address): it uses the address hipGetSymbolAddress returns for the
// current device, resolved once per device on the first call there.
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

static std::mutex g_scratch_mu;
static void *g_scratch_ptr[64];

static nh_status scratch_ptr(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(NH_ERR_HIP, "device id %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(NH_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return NH_OK;
}

nh_status bn_forward_train_noalloc(const void *x, void *y, nh_dtype io, int64_t N, int64_t C, int64_t HW,
                                   const float *gamma, const float *beta, float *running_mean,
                                   float *running_var, float momentum, float eps, float *stats, void *stream)
{
    if (!valid_dtype(io)) return fail(NH_ERR_DTYPE, "io dtype %d", (int)io);
    nh_status st = bn_check_shape(N, C, HW);
    if (st != NH_OK) return st;
    if (N * C * HW == 0) return ok();
    DeviceInfo d;
    if ((st = device_info(&d)) != NH_OK) return st;
    const size_t need = bn_ws_bytes(N, C, HW, d);
    if (need > kNoallocScratchBytes)
        return fail(NH_ERR_WORKSPACE,
                    "this shape needs %zu bytes of workspace; the allocation-free forward holds %zu bytes "
                    "(use bn_forward_train with a workspace)", need, kNoallocScratchBytes);
    void *ws = nullptr;
    if ((st = scratch_ptr(&ws)) != NH_OK) return st;
    return bn_forward_impl(0, x, y, io, N, C, HW, gamma, beta, running_mean, running_var, momentum, eps,
                           NH_ACT_NONE, 0.f, stats, ws, kNoallocScratchBytes, stream);
}

nh_status bn_forward_train_stage(int stage, const void *x, void *y, nh_dtype io, int64_t N, int64_t C,
                                 int64_t HW, const float *gamma, const float *beta, float *running_mean,
                                 float *running_var, float momentum, float eps, float *stats, void *ws,
                                 size_t ws_bytes, void *stream)
{
    if (stage != 1 && stage != 2) return fail(NH_ERR_ARG, "stage must be 1 or 2 (got %d)", stage);
    return bn_forward_impl(stage, x, y, io, N, C, HW, gamma, beta, running_mean, running_var, momentum, eps,
                           NH_ACT_NONE, 0.f, stats, ws, ws_bytes, stream);
}

nh_status bn_forward_train(const void *x, void *y, nh_dtype io, int64_t N, int64_t C, int64_t HW,
                           const float *gamma, const float *beta, float *running_mean,
                           float *running_var, float momentum, float eps, float *stats, void *ws,
                           size_t ws_bytes, void *stream)
{
    return bn_act_forward_train(x, y, io, N, C, HW, gamma, beta, running_mean, running_var, momentum,
                                eps, NH_ACT_NONE, 0.f, stats, ws, ws_bytes, stream);
}

// The BatchNorm training backward, whole (stage 0) or one of its two stages.
static nh_status bn_backward_impl(int stage, const void *dy, const void *x, nh_dtype io, int64_t N, int64_t C,
                                  int64_t HW, const float *stats, const float *beta, nh_act act, float slope,
                                  void *dx, float *grads, void *ws, size_t ws_bytes, void *stream)
{
    if (!valid_dtype(io)) return fail(NH_ERR_DTYPE, "io dtype %d", (int)io);
    nh_status st = bn_check_shape(N, C, HW);
    if (st != NH_OK) return st;
    if (N * C * HW == 0) return ok();
    if (!dy || !x || !stats || !grads) return fail(NH_ERR_NULL, "dy, x, stats and grads are required");
    if ((st = check_act(act, slope)) != NH_OK) return st;
    DeviceInfo d;
    if ((st = device_info(&d)) != NH_OK) return st;
    const size_t need = bn_ws_bytes(N, C, HW, d);
    if (!ws || ws_bytes < need || !aligned(ws, 16))
        return fail(NH_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned (got %zu)", need, ws_bytes);

    BnCall a{};
    bn_plan_grid(a, io, N, C, HW, bn_vec(io, HW, x, dy, dx), d);
    a.x = x;
    a.dy = dy;
    a.out = dx;
    a.beta = beta;
    a.act = act;
    a.slope = slope;
    a.stats = const_cast<float *>(stats);
    a.grads = grads;
    a.partials = static_cast<float *>(ws);
    a.stage = stage;
    bn_plan_training(a, d);
    if (bn_col_layout(io, HW, a.vec, a.channel_fused)) bn_col_plan(a, x, dy, dx);
    hipError_t e = bn_backward_launch(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "bn_backward launch");
    return ok();
}

nh_status bn_act_backward(const void *dy, const void *x, nh_dtype io, int64_t N, int64_t C, int64_t HW,
                          const float *stats, const float *beta, nh_act act, float slope, void *dx,
                          float *grads, void *ws, size_t ws_bytes, void *stream)
{
    return bn_backward_impl(0, dy, x, io, N, C, HW, stats, beta, act, slope, dx, grads, ws, ws_bytes, stream);
}

nh_status bn_backward_stage(int stage, const void *dy, const void *x, nh_dtype io, int64_t N, int64_t C,
                            int64_t HW, const float *stats, void *dx, float *grads, void *ws, size_t ws_bytes,
                            void *stream)
{
    if (stage != 1 && stage != 2) return fail(NH_ERR_ARG, "stage must be 1 or 2 (got %d)", stage);
    return bn_backward_impl(stage, dy, x, io, N, C, HW, stats, nullptr, NH_ACT_NONE, 0.f, dx, grads, ws,
                            ws_bytes, stream);
}

nh_status bn_backward(const void *dy, const void *x, nh_dtype io, int64_t N, int64_t C, int64_t HW,
                      const float *stats, void *dx, float *grads, void *ws, size_t ws_bytes,
                      void *stream)
{
    return bn_act_backward(dy, x, io, N, C, HW, stats, nullptr, NH_ACT_NONE, 0.f, dx, grads, ws,
                           ws_bytes, stream);
}

nh_status bn_forward_infer(const void *x, void *y, nh_dtype io, int64_t N, int64_t C, int64_t HW,
                           const float *gamma, const float *beta, const float *running_mean,
                           const float *running_var, float eps, nh_act act, float slope, void *stream)
{
    if (!valid_dtype(io)) return fail(NH_ERR_DTYPE, "io dtype %d", (int)io);
    nh_status st = bn_check_shape(N, C, HW);
    if (st != NH_OK) return st;
    if (N * C * HW == 0) return ok();
    if (!x || !y || !running_mean || !running_var)
        return fail(NH_ERR_NULL, "x, y, running_mean and running_var are required");
    if (!(eps >= 0.f) || !isfinite(eps)) return fail(NH_ERR_ARG, "eps must be finite and >= 0");
    if ((st = check_act(act, slope)) != NH_OK) return st;
    DeviceInfo d;
    if ((st = device_info(&d)) != NH_OK) return st;

    BnCall a{};
    bn_plan_grid(a, io, N, C, HW, bn_vec(io, HW, x, y, nullptr), d);
    a.inference = 1;
    a.x = x;
    a.out = y;
    a.gamma = gamma;
    a.beta = beta;
    a.running_mean = const_cast<float *>(running_mean);
    a.running_var = const_cast<float *>(running_var);
    a.eps = eps;
    a.act = act;
    a.slope = slope;
    if (bn_col_layout(io, HW, a.vec, 0)) bn_col_plan(a, x, y, nullptr);
    hipError_t e = bn_forward_launch(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "bn_forward_infer launch");
    return ok();
}

// ---- LayerNorm / RMSNorm ---------------------------------------------------------------
static nh_status rows_check_shape(int64_t rows, int64_t cols)
{
    if (rows < 0 || cols < 0) return fail(NH_ERR_SHAPE, "negative size (rows=%lld cols=%lld)",
                                          (long long)rows, (long long)cols);
    if (rows >= kMaxElems || cols >= kMaxElems || (rows > 0 && cols > 0 && rows * cols >= kMaxElems))
        return fail(NH_ERR_SHAPE, "rows*cols must be below 2^31");
    return NH_OK;
}

nh_status layernorm_backward_workspace(int64_t rows, int64_t cols, size_t *ws_bytes)
{
    if (!ws_bytes) return fail(NH_ERR_NULL, "ws_bytes is NULL");
    nh_status st = rows_check_shape(rows, cols);
    if (st != NH_OK) return st;
    if (rows * cols == 0) { *ws_bytes = 0; return ok(); }
    DeviceInfo d;
    if ((st = device_info(&d)) != NH_OK) return st;
    *ws_bytes = rows_ws_bytes(2, rows, cols, d);
    return ok();
}

nh_status rmsnorm_backward_workspace(int64_t rows, int64_t cols, size_t *ws_bytes)
{
    if (!ws_bytes) return fail(NH_ERR_NULL, "ws_bytes is NULL");
    nh_status st = rows_check_shape(rows, cols);
    if (st != NH_OK) return st;
    if (rows * cols == 0) { *ws_bytes = 0; return ok(); }
    DeviceInfo d;
    if ((st = device_info(&d)) != NH_OK) return st;
    *ws_bytes = rows_ws_bytes(1, rows, cols, d);
    return ok();
}

static nh_status rows_run(RowsCall &a, int Q, void *ws, size_t ws_bytes, void *stream)
{
    DeviceInfo d;
    nh_status st = device_info(&d);
    if (st != NH_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.rows == 0) {
        // No rows: the column sums are exact zeros; the finalize over zero
        // partial rows writes them.
        a.blocks = 0;
        a.partials = nullptr;
        a.dx = nullptr;
        a.maxg = 0;
        hipError_t e = rows_backward_launch(a, s);
        if (e != hipSuccess) return hip_fail(e, "rows finalize launch");
        return ok();
    }
    const size_t need = rows_ws_bytes(Q, a.rows, a.cols, d);
    if (!ws || ws_bytes < need || !aligned(ws, 16))
        return fail(NH_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned (got %zu)", need, ws_bytes);
    a.partials = static_cast<float *>(ws);
    bool vec_ok = true;
    auto need_align = [&](const void *p, int t) {
        if (!p) return;
        const size_t al = (size_t)a.vec * dtype_bytes(t);
        if (!aligned(p, al < 16 ? al : 16)) vec_ok = false;
    };
    need_align(a.x, a.x_t);
    need_align(a.dy, a.dy_t);
    need_align(a.dx, a.dx_t);
    need_align(a.w, a.w_t);
    if (a.kind == 2) {
        need_align(a.dresidual, NH_F32);
        need_align(a.dh, NH_F32);
        if (a.mask && !aligned(a.mask, (size_t)a.vec)) vec_ok = false;
    }
    RowsPlan p = rows_variant(a.cols, a.vec, vec_ok, a.kind == 2 ? kBdaMaxRowElems : kRowsMaxRowElems);
    a.depth = (int)g_override_rows_depth.load();
    a.colsum_cols = (int)g_override_colsum_cols.load();
    a.teams = (int)g_override_rows_teams.load();
    hipError_t e = hipSuccess;
    const bool vec_groups = vec_ok && a.cols % a.vec == 0;
    if (p.maxg == 0 || rows_narrow(a.cols, vec_groups ? a.vec : 1)) {
        rows_generic_plan(a, vec_ok, d);
        a.coef = a.gen_ct == 0
            ? reinterpret_cast<float *>(static_cast<char *>(ws) + rows_partials_bytes(Q, a.rows, a.cols, d))
            : nullptr;
        e = rows_backward_launch(a, s);
        if (e != hipSuccess) return hip_fail(e, "rows backward launch");
        return ok();
    }
    a.maxg = p.maxg;
    a.vec = p.vec;
    a.team = p.team;
    // Occupancy of the chosen variant, cached per device and variant.
    int dev = 0;
    (void)hipGetDevice(&dev);
    const int dxt = a.dx != nullptr ? a.dx_t : a.dy_t;
    const int64_t key = (((((((((int64_t)dev * 4 + a.kind) * 2 + a.x_t) * 2 + a.dy_t) * 2 + dxt) * 16 +
                           a.maxg) * 16 + a.vec) * 8 + a.depth) * 2 + (a.team == kWideTeam)) * 3 + a.teams;
    int occ = 0;
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        auto it = g_rows_occupancy.find(key);
        if (it != g_rows_occupancy.end()) occ = it->second;
    }
    if (occ == 0) {
        a.occupancy_out = &occ;
        e = rows_backward_launch(a, s);
        a.occupancy_out = nullptr;
        if (e != hipSuccess) return hip_fail(e, "row kernel occupancy query");
        std::lock_guard<std::mutex> lk(g_dev_mu);
        g_rows_occupancy[key] = occ;
    }
    rows_grid(p, a.kind, p.maxg * p.vec * (dtype_bytes(a.x_t) + dtype_bytes(a.dy_t)), a.cols / p.vec, a.rows,
              occ, d);
    a.blocks = p.blocks;
    e = rows_backward_launch(a, s);
    if (e != hipSuccess) return hip_fail(e, "rows backward launch");
    return ok();
}

nh_status layernorm_backward(const void *dy, nh_dtype dy_t, const void *x, nh_dtype x_t,
                             const float *mean, const float *rstd, const void *weight,
                             nh_dtype w_t, int64_t rows, int64_t cols, void *dx, nh_dtype dx_t,
                             void *dweight, void *dbias, void *ws, size_t ws_bytes, void *stream)
{
    if (!valid_dtype(dy_t) || !valid_dtype(x_t) || !valid_dtype(w_t) || !valid_dtype(dx_t))
        return fail(NH_ERR_DTYPE, "dtypes must be NH_F32 or NH_BF16");
    nh_status st = rows_check_shape(rows, cols);
    if (st != NH_OK) return st;
    if (cols == 0) return ok();
    if (rows > 0 && (!dy || !x || !mean || !rstd))
        return fail(NH_ERR_NULL, "dy, x, mean and rstd are required");
    RowsCall a{};
    a.kind = 0;
    a.x_t = x_t;
    a.dy_t = dy_t;
    a.w_t = w_t;
    a.dx_t = dx_t;
    a.rows = (int)rows;
    a.cols = (int)cols;
    a.vec = (x_t == NH_F32 || dy_t == NH_F32 || (dx && dx_t == NH_F32)) ? 4 : 8;
    a.x = x;
    a.dy = dy;
    a.w = weight;
    a.mean = mean;
    a.rstd = rstd;
    a.dx = dx;
    a.dweight = dweight;
    a.dbias = dbias;
    return rows_run(a, 2, ws, ws_bytes, stream);
}

nh_status bda_layernorm_backward_workspace(int64_t rows, int64_t cols, size_t *ws_bytes)
{
    if (!ws_bytes) return fail(NH_ERR_NULL, "ws_bytes is NULL");
    nh_status st = rows_check_shape(rows, cols);
    if (st != NH_OK) return st;
    if (rows * cols == 0) { *ws_bytes = 0; return ok(); }
    DeviceInfo d;
    if ((st = device_info(&d)) != NH_OK) return st;
    *ws_bytes = rows_ws_bytes(3, rows, cols, d);
    return ok();
}

nh_status bda_layernorm_backward(const void *dy, nh_dtype dy_t, const void *x, nh_dtype x_t,
                                 const float *mean, const float *rstd, const void *weight,
                                 nh_dtype w_t, const float *dresidual, const uint8_t *mask,
                                 float scale, int64_t rows, int64_t cols, float *dh, void *da,
                                 void *dweight, void *dbias, void *dbias_in, void *ws,
                                 size_t ws_bytes, void *stream)
{
    if (!valid_dtype(dy_t) || !valid_dtype(x_t) || !valid_dtype(w_t))
        return fail(NH_ERR_DTYPE, "dtypes must be NH_F32 or NH_BF16");
    nh_status st = rows_check_shape(rows, cols);
    if (st != NH_OK) return st;
    if (cols == 0) return ok();
    if (rows > 0 && (!dy || !x || !mean || !rstd))
        return fail(NH_ERR_NULL, "dy, x, mean and rstd are required");
    if (!isfinite(scale)) return fail(NH_ERR_ARG, "scale must be finite");
    RowsCall a{};
    a.kind = 2;
    a.x_t = x_t;
    a.dy_t = dy_t;
    a.w_t = w_t;
    a.dx_t = dy_t;
    a.rows = (int)rows;
    a.cols = (int)cols;
    a.vec = (x_t == NH_F32 || dy_t == NH_F32) ? 4 : 8;
    a.x = x;
    a.dy = dy;
    a.w = weight;
    a.mean = mean;
    a.rstd = rstd;
    a.dx = da;
    a.dresidual = dresidual;
    a.mask = mask;
    a.scale = scale;
    a.dh = dh;
    a.dweight = dweight;
    a.dbias = dbias;
    a.dbias_in = dbias_in;
    return rows_run(a, 3, ws, ws_bytes, stream);
}

nh_status rmsnorm_backward(const void *dy, const void *x, nh_dtype t, const float *rms, float eps,
                           const void *weight, int64_t rows, int64_t cols, void *dx, void *dweight,
                           void *ws, size_t ws_bytes, void *stream)
{
    if (!valid_dtype(t)) return fail(NH_ERR_DTYPE, "dtype must be NH_F32 or NH_BF16");
    nh_status st = rows_check_shape(rows, cols);
    if (st != NH_OK) return st;
    if (cols == 0) return ok();
    if (rows > 0 && (!dy || !x)) return fail(NH_ERR_NULL, "dy and x are required");
    if (!rms && (!(eps >= 0.f) || !isfinite(eps)))
        return fail(NH_ERR_ARG, "eps must be finite and >= 0 when rms is recomputed");
    RowsCall a{};
    a.kind = 1;
    a.x_t = a.dy_t = a.dx_t = a.w_t = t;
    a.rows = (int)rows;
    a.cols = (int)cols;
    a.vec = t == NH_F32 ? 4 : 8;
    a.x = x;
    a.dy = dy;
    a.w = weight;
    a.rms = rms;
    a.eps = eps;
    a.dx = dx;
    a.dweight = dweight;
    return rows_run(a, 1, ws, ws_bytes, stream);
}

// ---- LayerNorm / RMSNorm forward ----------------------------------------------------------
static nh_status rows_forward_run(FwdCall &a, void *stream)
{
    DeviceInfo d;
    nh_status st = device_info(&d);
    if (st != NH_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    bool vec_ok = true;
    auto need_align = [&](const void *p, int t) {
        if (!p) return;
        const size_t al = (size_t)a.vec * dtype_bytes(t);
        if (!aligned(p, al < 16 ? al : 16)) vec_ok = false;
    };
    need_align(a.x, a.x_t);
    need_align(a.y, a.y_t);
    need_align(a.w, a.w_t);
    need_align(a.b, a.w_t);
    RowsPlan p = rows_variant(a.cols, a.vec, vec_ok);
    a.depth = (int)g_override_rows_depth.load();
    hipError_t e = hipSuccess;
    const bool vec_groups = vec_ok && a.cols % a.vec == 0;
    if (p.maxg == 0 || rows_narrow(a.cols, vec_groups ? a.vec : 1)) {
        rows_forward_generic_plan(a, vec_ok, d);
        e = rows_forward_launch(a, s);
        if (e != hipSuccess) return hip_fail(e, "forward row kernel launch");
        return ok();
    }
    a.maxg = p.maxg;
    a.vec = p.vec;
    a.team = p.team;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const int64_t key = -1 - (((((((((int64_t)dev * 2 + a.kind) * 2 + a.x_t) * 2 + a.y_t) * 16 + a.maxg) * 16) +
                                a.vec) * 8 + a.depth) * 2 + (a.team == kWideTeam));
    int occ = 0;
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        auto it = g_rows_occupancy.find(key);
        if (it != g_rows_occupancy.end()) occ = it->second;
    }
    if (occ == 0) {
        a.occupancy_out = &occ;
        e = rows_forward_launch(a, s);
        a.occupancy_out = nullptr;
        if (e != hipSuccess) return hip_fail(e, "forward row kernel occupancy query");
        std::lock_guard<std::mutex> lk(g_dev_mu);
        g_rows_occupancy[key] = occ;
    }
    // No column partials in the forward: fill the device (at most 8 blocks per CU).
    int64_t g = (int64_t)d.cus * (occ < 1 ? 1 : (occ > 8 ? 8 : occ));
    if (g > a.rows) g = a.rows;
    a.blocks = (int)g;
    e = rows_forward_launch(a, s);
    if (e != hipSuccess) return hip_fail(e, "forward row kernel launch");
    return ok();
}

nh_status layernorm_forward(const void *x, nh_dtype x_t, const void *weight, const void *bias,
                            nh_dtype w_t, int64_t rows, int64_t cols, float eps, void *y,
                            nh_dtype y_t, float *mean, float *rstd, void *stream)
{
    if (!valid_dtype(x_t) || !valid_dtype(w_t) || !valid_dtype(y_t))
        return fail(NH_ERR_DTYPE, "dtypes must be NH_F32 or NH_BF16");
    nh_status st = rows_check_shape(rows, cols);
    if (st != NH_OK) return st;
    if (rows * cols == 0) return ok();
    if (!x || !y || !mean) return fail(NH_ERR_NULL, "x, y and mean are required");
    if (!(eps >= 0.f) || !isfinite(eps)) return fail(NH_ERR_ARG, "eps must be finite and >= 0");
    FwdCall a{};
    a.kind = 0;
    a.x_t = x_t;
    a.y_t = y_t;
    a.w_t = w_t;
    a.rows = (int)rows;
    a.cols = (int)cols;
    a.vec = (x_t == NH_F32 || y_t == NH_F32) ? 4 : 8;
    a.x = x;
    a.w = weight;
    a.b = bias;
    a.eps = eps;
    a.y = y;
    a.stat0 = mean;
    a.stat1 = rstd;
    return rows_forward_run(a, stream);
}

nh_status rmsnorm_forward(const void *x, nh_dtype t, const void *weight, int64_t rows, int64_t cols,
                          float eps, void *y, float *rms, void *stream)
{
    if (!valid_dtype(t)) return fail(NH_ERR_DTYPE, "dtype must be NH_F32 or NH_BF16");
    nh_status st = rows_check_shape(rows, cols);
    if (st != NH_OK) return st;
    if (rows * cols == 0) return ok();
    if (!x || !y) return fail(NH_ERR_NULL, "x and y are required");
    if (!(eps >= 0.f) || !isfinite(eps)) return fail(NH_ERR_ARG, "eps must be finite and >= 0");
    FwdCall a{};
    a.kind = 1;
    a.x_t = a.y_t = a.w_t = t;
    a.rows = (int)rows;
    a.cols = (int)cols;
    a.vec = t == NH_F32 ? 4 : 8;
    a.x = x;
    a.w = weight;
    a.y = y;
    a.eps = eps;
    a.stat0 = rms;
    return rows_forward_run(a, stream);
}

// ---- measurement -------------------------------------------------------------------------
nh_status nh_timing_enable(int on)
{
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (on) {
        g_records.clear();
        g_pool_used = 0;
    }
    g_timing.store(on != 0);
    return ok();
}

nh_status nh_timing_reserve(int64_t launches)
{
    if (launches < 0) return fail(NH_ERR_ARG, "launches must be >= 0");
    std::lock_guard<std::mutex> lk(g_timing_mu);
    while ((int64_t)g_event_pool.size() < 2 * launches) {
        hipEvent_t e = nullptr;
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) return hip_fail(err, "hipEventCreate");
        g_event_pool.push_back(e);
    }
    return ok();
}

nh_status nh_timing_read(int kernel, double *total_ms, int64_t *launches)
{
    if (kernel < 0 || kernel >= NH_K_COUNT) return fail(NH_ERR_ARG, "kernel id %d", kernel);
    if (!total_ms || !launches) return fail(NH_ERR_NULL, "total_ms and launches are required");
    std::lock_guard<std::mutex> lk(g_timing_mu);
    double tot = 0.0;
    int64_t n = 0;
    for (const TimingRec &r : g_records) {
        if (r.kid != kernel) continue;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        tot += ms;
        ++n;
    }
    *total_ms = tot;
    *launches = n;
    return ok();
}

nh_status nh_calib_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    if (bytes == 0) return ok();
    if (!src || !dst) return fail(NH_ERR_NULL, "src and dst are required");
    DeviceInfo d;
    nh_status st = device_info(&d);
    if (st != NH_OK) return st;
    hipError_t e = calib_copy_launch(src, dst, bytes, (int)bn_slots(d), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "nh_calib_copy launch");
    return ok();
}

nh_status nh_calib_read(const float *a, int64_t n, float *block_sums, int64_t max_blocks, void *stream)
{
    if (n < 0 || max_blocks < 0) return fail(NH_ERR_SHAPE, "negative size");
    if (n == 0) return ok();
    if (!a || !block_sums) return fail(NH_ERR_NULL, "a and block_sums are required");
    if (n % 4 != 0 || !aligned(a, 16)) return fail(NH_ERR_SHAPE, "n must be a multiple of 4, a 16-byte aligned");
    if (max_blocks < 1) return fail(NH_ERR_SHAPE, "max_blocks must be >= 1");
    DeviceInfo d;
    nh_status st = device_info(&d);
    if (st != NH_OK) return st;
    hipError_t e = calib_read_launch(a, n, block_sums, max_blocks, (int)bn_slots(d),
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "nh_calib_read launch");
    return ok();
}

nh_status nh_calib_add(const float *a, const float *b, float *out, int64_t n, void *stream)
{
    if (n < 0) return fail(NH_ERR_SHAPE, "negative n");
    if (n == 0) return ok();
    if (!a || !b || !out) return fail(NH_ERR_NULL, "a, b and out are required");
    DeviceInfo d;
    nh_status st = device_info(&d);
    if (st != NH_OK) return st;
    hipError_t e = calib_add_launch(a, b, out, n, (int)bn_slots(d), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "nh_calib_add launch");
    return ok();
}

nh_status nh_bn_plan(int64_t N, int64_t C, int64_t HW, nh_dtype io, int *grid_y)
{
    if (!grid_y) return fail(NH_ERR_NULL, "grid_y is NULL");
    if (!valid_dtype(io)) return fail(NH_ERR_DTYPE, "io dtype %d", (int)io);
    nh_status st = bn_check_shape(N, C, HW);
    if (st != NH_OK) return st;
    if (N * C * HW == 0) { *grid_y = 0; return ok(); }
    DeviceInfo d;
    if ((st = device_info(&d)) != NH_OK) return st;
    const int v = bn_vec(io, HW, nullptr, nullptr, nullptr);
    *grid_y = (int)bn_grid_y_for(N * (HW / v), C, d);
    return ok();
}

nh_status nh_rows_plan(int64_t rows, int64_t cols, int *blocks)
{
    if (!blocks) return fail(NH_ERR_NULL, "blocks is NULL");
    nh_status st = rows_check_shape(rows, cols);
    if (st != NH_OK) return st;
    if (rows * cols == 0) { *blocks = 0; return ok(); }
    DeviceInfo d;
    if ((st = device_info(&d)) != NH_OK) return st;
    *blocks = (int)rows_partial_rows(rows, cols, d);
    return ok();
}

nh_status nh_plan_override(const char *key, int64_t value)
{
    if (!key) return fail(NH_ERR_NULL, "key is NULL");
    if (value < 0) return fail(NH_ERR_ARG, "value must be >= 0");
    if (strcmp(key, "bn_grid_y") == 0) g_override_bn_grid_y.store(value);
    else if (strcmp(key, "bn_ew_grid_y") == 0) g_override_bn_ew_grid_y.store(value);
    else if (strcmp(key, "rows_blocks") == 0) g_override_rows_blocks.store(value);
    else if (strcmp(key, "rows_depth") == 0) {
        if (value < 0 || value > 4) return fail(NH_ERR_ARG, "rows_depth must be 0..4");
        g_override_rows_depth.store(value);
    }
    else if (strcmp(key, "colsum_cols") == 0) {
        if (value != 0 && value != 8 && value != 16 && value != 32 && value != 64)
            return fail(NH_ERR_ARG, "colsum_cols must be 0, 8, 16, 32 or 64");
        g_override_colsum_cols.store(value);
    }
    else if (strcmp(key, "bn_layout") == 0) {
        if (value > 2) return fail(NH_ERR_ARG, "bn_layout must be 0, 1 or 2");
        g_override_bn_layout.store(value);
    }
    else if (strcmp(key, "bn_channel") == 0) {
        if (value > 2) return fail(NH_ERR_ARG, "bn_channel must be 0, 1 or 2");
        g_override_bn_channel.store(value);
    }
    else if (strcmp(key, "bn_channel_threads") == 0) {
        if (value != 0 && value != kBnThreads && value != kBnChannelBigBlock)
            return fail(NH_ERR_ARG, "bn_channel_threads must be 0, %d or %d", kBnThreads, kBnChannelBigBlock);
        g_override_bn_channel_threads.store(value);
    }
    else if (strcmp(key, "rows_narrow") == 0) {
        if (value > 1) return fail(NH_ERR_ARG, "rows_narrow must be 0 or 1");
        g_override_rows_narrow.store(value);
    }
    else if (strcmp(key, "rows_teams") == 0) {
        if (value > 2) return fail(NH_ERR_ARG, "rows_teams must be 0, 1 or 2");
        g_override_rows_teams.store(value);
    }
    else if (strcmp(key, "bn_finalize_kernels") == 0) g_override_bn_finalize_kernels.store(value);
    else if (strcmp(key, "bn_block_order") == 0) {
        if (value > 2) return fail(NH_ERR_ARG, "bn_block_order must be 0, 1 or 2");
        g_override_bn_block_order.store(value);
    }
    else if (strcmp(key, "bn_unit_order") == 0) {
        if (value > 2) return fail(NH_ERR_ARG, "bn_unit_order must be 0, 1 or 2");
        g_override_bn_unit_order.store(value);
    }
    else return fail(NH_ERR_ARG, "unknown override key '%s'", key);
    return ok();
}

nh_status nh_selftest_host(void)
{
    // Fast division: exhaustive over small divisors and dividends, plus edges.
    for (uint32_t d = 1; d <= 4096; ++d) {
        const FastDiv f = make_fastdiv(d);
        for (uint32_t n = 0; n < 20000; ++n)
            if (f.div(n) != n / d) return fail(NH_ERR_ARG, "fastdiv %u/%u", n, d);
        const uint32_t edges[] = {0x7fffffffu, 0x7ffffffeu, 0x40000000u, 0x3fffffffu,
                                  d * 1000u - 1u, d * 1000u, d * 1000u + 1u};
        for (uint32_t n : edges)
            if (n < 0x80000000u && f.div(n) != n / d) return fail(NH_ERR_ARG, "fastdiv %u/%u", n, d);
    }
    uint64_t s = 0x9e3779b97f4a7c15ull;
    for (int i = 0; i < 2000000; ++i) {
        s ^= s << 13; s ^= s >> 7; s ^= s << 17;
        const uint32_t d = (uint32_t)(s % 0x7fffffffull) + 1u;
        const uint32_t n = (uint32_t)((s >> 32) & 0x7fffffffu);
        if (make_fastdiv(d).div(n) != n / d) return fail(NH_ERR_ARG, "fastdiv %u/%u", n, d);
    }
    // BatchNorm grid.  Contiguous: within [1, slots/C] (at least 1), and
    // enough blocks to fill the slots whenever the channel has the work for
    // them.  Interleaved: the contiguous grid where a block would get less
    // than a whole sweep; else within [that grid, 2*slots/C] with a whole
    // sweep for every block, and the contiguous grid itself where two rounds
    // would exceed kBnTwoRoundMaxGrid blocks per channel.  Both never decrease with the unit count (the
    // workspace query sizes the partials for the largest unit count a shape
    // can take).
    const int64_t slots = 2048;
    const int64_t Cs[] = {1, 3, 32, 37, 256, 2048, 5000};
    const int64_t Us[] = {1, 100, 1023, 1024, 65536, 1 << 20, 25088, 6272, 100352};
    for (int64_t C : Cs)
        for (int64_t u : Us) {
            const int64_t g = bn_auto_grid_y(u, C, slots, false);
            const int64_t gi = bn_auto_grid_y(u, C, slots, true);
            const int64_t cap = slots / C > 1 ? slots / C : 1;
            if (g < 1 || g > cap || g > u) return fail(NH_ERR_ARG, "bn grid %lld for C=%lld u=%lld",
                                                      (long long)g, (long long)C, (long long)u);
            if (u >= cap * kBnGridMinUnits && g != cap)
                return fail(NH_ERR_ARG, "bn grid underfills: %lld", (long long)g);
            if (u < g * kBnMinUnits ? gi != g
                                    : (gi < g || gi > 2 * cap || gi * kBnMinUnits > u ||
                                       (2 * cap > kBnTwoRoundMaxGrid && gi != g)))
                return fail(NH_ERR_ARG, "bn interleaved grid %lld for C=%lld u=%lld", (long long)gi,
                            (long long)C, (long long)u);
            for (bool il : {false, true})
                if (bn_auto_grid_y(u + 1, C, slots, il) < bn_auto_grid_y(u, C, slots, il))
                    return fail(NH_ERR_ARG, "bn grid decreases at C=%lld u=%lld", (long long)C, (long long)u);
        }
    // BatchNorm unit walk at the largest shapes the ABI accepts: for every
    // block, the unsigned loop index (up to a stride past the block's last
    // unit) must not wrap, and the first and last unit of every block (of the
    // first and last channel) must map inside the tensor, at the offset the
    // plain division gives.
    struct MaxShape { int N, C, HW, vec; };
    const MaxShape shapes[] = {
        {1, 1, 0x7fffffff, 1},                 // one channel of 2^31 - 1 elements, scalar units
        {1, 2, 0x3fffffff, 1},                 // 2 channels, odd planes
        {2, 4, (1 << 28) - 8, 8},              // bf16 vector units
        {2, 4, (1 << 28) - 8, 4},              // fp32 vector units
        {16384, 3, 43690, 1},                  // many planes per channel
    };
    for (const MaxShape &m : shapes) {
        const int64_t total = (int64_t)m.N * m.C * m.HW;
        if (total >= kMaxElems) return fail(NH_ERR_ARG, "max shape exceeds the element limit");
        const int64_t units = (int64_t)m.N * (m.HW / m.vec);
        // one block per channel, the planned split, and 2048 blocks per channel
        for (int64_t grid_y : {(int64_t)1, bn_auto_grid_y(units, m.C, slots, true),
                               std::min<int64_t>(units, 2048)}) {
          for (int ilv = 0; ilv < 2; ++ilv) {
            const BnGeom g = make_bn_geom(m.N, m.C, m.HW, m.vec, (int)grid_y, 0, ilv);
            const uint64_t sweep = (uint64_t)kBnMinUnits;
            for (int c = 0; c < m.C; c += (m.C > 1 ? m.C - 1 : 1)) {
                for (int yb = 0; yb < g.grid_y; ++yb) {
                    // bn_range in 64-bit arithmetic: the 32-bit forms must not wrap
                    // for any index the loops form (up to a step past u1).
                    const uint64_t c0 = (uint64_t)yb * (uint64_t)g.upb;
                    const uint64_t u0 = ilv ? (uint64_t)yb * sweep : c0;
                    const uint64_t u1 = ilv ? (uint64_t)g.units : std::min<uint64_t>(c0 + (uint64_t)g.upb, (uint64_t)g.units);
                    const uint64_t step = ilv ? (uint64_t)g.grid_y * sweep : sweep;
                    if (c0 + (uint64_t)g.upb >= (1ull << 32) || u0 >= (1ull << 32) || u1 + step >= (1ull << 32))
                        return fail(NH_ERR_ARG, "bn unit index wraps (C=%d yb=%d)", c, yb);
                    if (u0 >= u1) continue;
                    const uint32_t probe[] = {(uint32_t)u0, (uint32_t)(u1 - 1)};
                    for (uint32_t u : probe) {
                        const int64_t off = m.vec == 1 ? bn_unit_offset<1>(g, c, u)
                                            : (m.vec == 4 ? bn_unit_offset<4>(g, c, u) : bn_unit_offset<8>(g, c, u));
                        const int64_t n = u / (uint32_t)g.HWv, j = u % (uint32_t)g.HWv;
                        if (off != (n * m.C + c) * m.HW + j * m.vec || off < 0 || off + m.vec > total)
                            return fail(NH_ERR_ARG, "bn unit offset out of range (u=%u)", u);
                    }
                }
            }
          }
        }
    }
    // BatchNorm row layout: the chunks cover the rows exactly once, within the
    // workspace's chunks; the column lanes are a power of two of at most
    // kBnColLanes that, with the row lanes, make one block; the strips cover
    // the row length; block ids map one to one onto (strip, chunk).
    {
        const int64_t Ns[] = {1, 2, 15, 16, 17, 255, 1000, 4097, 65536, 200704, 1 << 20};
        const int64_t Ls[][2] = {{1, 1},   {3, 1},    {8, 1},     {64, 1},  {256, 1}, {1000, 1},
                                 {4096, 1}, {37, 4}, {256, 16}, {2048, 49}, {5, 3}};
        std::vector<int> seen;
        for (int64_t n : Ns)
            for (const auto &cl : Ls)
                for (int vec : {1, 4, 8}) {
                    const int64_t C = cl[0], HW = cl[1];
                    if ((C * HW) % vec != 0 || n * C * HW >= kMaxElems) continue;
                    const BnColGeom g = make_bn_col_geom((int)n, (int)C, (int)HW, vec);
                    const int64_t lanes = (int64_t)1 << g.cl_log2;
                    bool bad = g.rb < 1 || g.rpc < 1 || (int64_t)g.rb * g.rpc < n ||
                               (int64_t)(g.rb - 1) * g.rpc >= n || g.rb > bn_col_chunks_max(n, C * HW) ||
                               lanes > kBnColLanes || lanes * g.rl != kBnThreads ||
                               g.strips * lanes * vec < C * HW || (int64_t)(g.strips - 1) * lanes * vec >= C * HW ||
                               g.L != C * HW;
                    if (!bad) {
                        const int total = g.strips * g.rb;
                        seen.assign((size_t)total, 0);
                        for (int id = 0; id < total && !bad; ++id) {
                            const BnColWork w = bn_col_work(g, id);
                            const int64_t k = (int64_t)w.chunk * g.strips + w.strip;
                            bad = w.strip < 0 || w.strip >= g.strips || w.chunk < 0 || w.chunk >= g.rb ||
                                  seen[(size_t)k]++ != 0;
                        }
                    }
                    if (bad)
                        return fail(NH_ERR_ARG, "bn row-layout plan (N=%lld C=%lld HW=%lld vec=%d)", (long long)n,
                                    (long long)C, (long long)HW, vec);
                }
    }
    // Generic row plan, on a 256-CU device: the blocks fit the workspace's
    // partial rows, the chunks cover the rows exactly once, the strips cover
    // the columns, the grid is launchable and the coefficient region exists.
    DeviceInfo dv;
    dv.valid = true;
    dv.cus = 256;
    const int64_t Rs[] = {1, 2, 31, 33, 97, 1000, 4097, 65537, (1 << 18) - 1, 33554431};
    const int64_t Hs[] = {1, 2, 3, 8, 31, 63, 64, 65, 128, 256, 257, 512, 1000, 1601, 4096, 16385, 32768,
                          65536, 1 << 20};
    for (int64_t rows : Rs)
        for (int64_t cols : Hs) {
            if (rows * cols >= kMaxElems) continue;
            for (int vec : {4, 8})
                for (bool vec_ok : {false, true}) {
                    RowsCall a{};
                    a.rows = (int)rows;
                    a.cols = (int)cols;
                    a.vec = vec;
                    rows_generic_plan(a, vec_ok, dv);
                    const int64_t gmax = rows_partial_rows(rows, cols, dv);
                    if (a.blocks < 1 || a.blocks > gmax)
                        return fail(NH_ERR_ARG, "generic blocks %d (rows=%lld cols=%lld)", a.blocks,
                                    (long long)rows, (long long)cols);
                    if (a.gen_ct > 0) {
                        const bool vec_fits = vec_ok && cols % vec == 0;
                        if ((a.vec != 1 && (a.vec != vec || !vec_fits)) || cols % a.vec != 0 ||
                            cols / a.vec > kGenNarrowGroups || a.gen_ct < cols / a.vec ||
                            a.gen_ct > kGenNarrowGroups || (a.gen_ct & (a.gen_ct - 1)) != 0 ||
                            (vec_fits && a.vec == 1))
                            return fail(NH_ERR_ARG, "narrow plan ct=%d vec=%d cols=%lld", a.gen_ct, a.vec,
                                        (long long)cols);
                        continue;
                    }
                    const int64_t rpc = a.gen_rpc;
                    const int64_t strips = ceil_div(cols / a.vec, kGenStripGroups);
                    if (cols <= kGenNarrowGroups || rpc < 1 || (int64_t)(a.blocks - 1) * rpc >= rows ||
                        (int64_t)a.blocks * rpc < rows || cols % a.vec != 0 ||
                        (a.vec != 1 && (!vec_ok || a.vec != vec)) ||
                        strips * kGenStripGroups * a.vec < cols || strips >= (1ll << 31) || a.blocks > 65535 ||
                        (a.gen_coef_waves != 1 && a.gen_coef_waves != kGenCoefTeamWaves) ||
                        a.gen_coef_segs < 1 || a.gen_coef_segs > gen_coef_slots(rows) ||
                        (a.gen_coef_waves == 1 && a.gen_coef_segs != 1) ||
                        (a.gen_coef_segs > 1 && (cols / a.vec) / a.gen_coef_segs < kGenCoefMinSegGroups) ||
                        rows * a.gen_coef_segs >= (1ll << 31))
                        return fail(NH_ERR_ARG, "strip plan rpc=%lld blocks=%d (rows=%lld cols=%lld)",
                                    (long long)rpc, a.blocks, (long long)rows, (long long)cols);
                    for (int Q = 1; Q <= 3; ++Q)
                        if (rows_ws_bytes(Q, rows, cols, dv) <
                            rows_partials_bytes(Q, rows, cols, dv) + (size_t)rows * a.gen_coef_segs * 2 * sizeof(float) ||
                            rows_partials_bytes(Q, rows, cols, dv) < (size_t)Q * a.blocks * cols * sizeof(float))
                            return fail(NH_ERR_ARG, "generic workspace too small (rows=%lld cols=%lld)",
                                        (long long)rows, (long long)cols);
                }
        }
    return ok();
}

} // extern "C"
