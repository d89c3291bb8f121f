// C ABI of the indexer library: argument checks (host only, before any HIP
// call), plan choice, and kernel dispatch.  See include/csa_index.h.
#include "csa_index.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "csa_backward.hpp"
#include "csa_launch.hpp"

namespace {

thread_local std::string g_last_error;

csa_status fail(csa_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

csa_status ok()
{
    g_last_error.clear();
    return CSA_OK;
}

constexpr int kMaxTopK = 2048;
constexpr int kMaxW = 1 << 30;
constexpr int kNumCUs = 256; // MI355X; only used to choose a plan
constexpr int64_t kMaxKeyStride = int64_t(1) << 24;
// A row-tile launch with fewer workgroups than this leaves the chip idle.
constexpr int64_t kMinRowBlocks = 2 * kNumCUs;
// Rows shorter than this are not worth splitting.
constexpr int kMinSplitW = 2048;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// 32-head MFMA blocks, rounded up to a power of two (1, 2 or 4).
int head_blocks(int H)
{
    int hb = (H + 31) / 32;
    int p = 1;
    while (p < hb)
        p <<= 1;
    return p;
}

struct Checked {
    int64_t rows = 0; // B*S
    int HB = 0;
    int plan = 0;
};

csa_status check_problem(const csa_index_problem *p, Checked &c)
{
    if (!p)
        return fail(CSA_ERR_INVALID_ARG, "problem descriptor is NULL");
    if (p->B < 0 || p->S < 0 || p->W < 0)
        return fail(CSA_ERR_INVALID_ARG, "negative size (B=%d S=%d W=%d)", p->B, p->S, p->W);
    if (p->H < 1 || p->D < 1)
        return fail(CSA_ERR_INVALID_ARG, "H and D must be >= 1 (H=%d D=%d)", p->H, p->D);
    if (p->compress_rate < 1)
        return fail(CSA_ERR_INVALID_ARG, "compress_rate must be >= 1 (got %d)", p->compress_rate);
    if (!std::isfinite(p->scale))
        return fail(CSA_ERR_INVALID_ARG, "scale must be finite");
    if (p->plan < CSA_PLAN_AUTO || p->plan > CSA_PLAN_SPLIT_ROWS)
        return fail(CSA_ERR_INVALID_ARG, "unknown plan %d", p->plan);
    if (p->D != 32 && p->D != 64 && p->D != 128)
        return fail(CSA_ERR_UNSUPPORTED, "D=%d not implemented (D must be 32, 64 or 128)", p->D);
    if (p->H > 128)
        return fail(CSA_ERR_UNSUPPORTED, "H=%d not implemented (H <= 128)", p->H);
    if (p->W > kMaxW)
        return fail(CSA_ERR_UNSUPPORTED, "W=%d above the supported maximum %d", p->W, kMaxW);
    if (p->q_sb < 0 || p->q_sh < 0 || p->q_ss < 0 || p->k_sb < 0 || p->k_sw < 0 || p->w_sb < 0 || p->w_ss < 0)
        return fail(CSA_ERR_INVALID_ARG, "strides must be non-negative");
    if ((p->q_sb | p->q_sh | p->q_ss | p->k_sb | p->k_sw) % 8 != 0)
        return fail(CSA_ERR_UNSUPPORTED, "q and k strides must be multiples of 8 elements (16-byte rows)");
    if (p->k_sw >= kMaxKeyStride)
        return fail(CSA_ERR_UNSUPPORTED, "k_sw=%lld not below %lld (key tiles are addressed with 32-bit offsets)",
                    (long long)p->k_sw, (long long)kMaxKeyStride);
    c.rows = (int64_t)p->B * p->S;
    c.HB = head_blocks(p->H);
    // sizes up to INT32_MAX: ceiling divisions in 64 bits
    int64_t row_blocks = (int64_t)p->B * (((int64_t)p->S + csa::kRowsPerBlock - 1) / csa::kRowsPerBlock);
    int plan = p->plan;
    if (plan == CSA_PLAN_AUTO)
        plan = ((row_blocks < kMinRowBlocks && p->W >= kMinSplitW) || p->W > csa::kRowTilesMaxW)
                   ? CSA_PLAN_SPLIT_ROWS
                   : CSA_PLAN_ROW_TILES;
    if (plan == CSA_PLAN_ROW_TILES && p->W > csa::kRowTilesMaxW)
        return fail(CSA_ERR_UNSUPPORTED, "the row-tile plan takes W <= %d (got %d)", csa::kRowTilesMaxW, p->W);
    c.plan = plan;
    // grid sizes must fit a 32-bit launch
    int64_t chunks = ((int64_t)p->W + csa::kSplitChunk - 1) / csa::kSplitChunk;
    if (row_blocks > 0x7FFFFFFF || c.rows * (chunks > 0 ? chunks : 1) > 0x7FFFFFFF)
        return fail(CSA_ERR_UNSUPPORTED, "problem too large for one launch");
    return CSA_OK;
}

csa_status check_inputs(const csa_index_problem *p, const Checked &c, const void *q, const void *k, const void *w,
                        const csa_index_masks *masks)
{
    if (c.rows > 0) {
        if (!q || !w)
            return fail(CSA_ERR_INVALID_ARG, "q and w must be non-NULL");
        if (!aligned(q, 16))
            return fail(CSA_ERR_INVALID_ARG, "q must be 16-byte aligned");
        if (!aligned(w, 2))
            return fail(CSA_ERR_INVALID_ARG, "w must be 2-byte aligned");
    }
    if ((int64_t)p->B * p->W > 0) {
        if (!k)
            return fail(CSA_ERR_INVALID_ARG, "k must be non-NULL");
        if (!aligned(k, 16))
            return fail(CSA_ERR_INVALID_ARG, "k must be 16-byte aligned");
    }
    if (masks) {
        if ((masks->q_seg == nullptr) != (masks->k_seg == nullptr))
            return fail(CSA_ERR_INVALID_ARG, "q_seg and k_seg must be both NULL or both set");
        if (!aligned(masks->q_offset, 4) || !aligned(masks->q_seg, 4) || !aligned(masks->k_seg, 4))
            return fail(CSA_ERR_INVALID_ARG, "mask arrays must be 4-byte aligned");
    }
    return CSA_OK;
}

csa::KernelArgs make_args(const csa_index_problem *p, const Checked &c, const void *q, const void *k, const void *w,
                          const csa_index_masks *masks)
{
    csa::KernelArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.w = static_cast<const uint16_t *>(w);
    if (masks) {
        a.q_offset = masks->q_offset;
        a.q_seg = masks->q_seg;
        a.k_seg = masks->k_seg;
    }
    a.q_sb = p->q_sb;
    a.q_sh = p->q_sh;
    a.q_ss = p->q_ss;
    a.k_sb = p->k_sb;
    a.k_sw = p->k_sw;
    a.w_sb = p->w_sb;
    a.w_ss = p->w_ss;
    a.rows = c.rows;
    a.B = p->B;
    a.S = p->S;
    a.H = p->H;
    a.W = p->W;
    a.m = p->compress_rate;
    a.scale = p->scale;
    a.n_row_blocks = (int)(((int64_t)p->S + csa::kRowsPerBlock - 1) / csa::kRowsPerBlock);
    a.n_chunks = (int)(((int64_t)p->W + csa::kSplitChunk - 1) / csa::kSplitChunk);
    return a;
}

// Device properties the host code needs (LDS per workgroup, compute units),
// queried once per device and kept for the life of the process.
struct DeviceInfo {
    int lds = 0;
    int cus = 0;
    hipError_t err = hipSuccess;
};

constexpr int kMaxDevices = 64;
std::mutex g_info_mutex;
std::atomic<bool> g_info_ready[kMaxDevices];
DeviceInfo g_info[kMaxDevices]; // written once, under the mutex, before its flag is set

DeviceInfo query_device(int dev)
{
    DeviceInfo d;
    d.err = hipDeviceGetAttribute(&d.lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (d.err == hipSuccess)
        d.err = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
    return d;
}

// Properties of the calling thread's current device.
csa_status current_device(DeviceInfo &out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(CSA_ERR_DEVICE, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) {
        out = query_device(dev);
    } else if (g_info_ready[dev].load(std::memory_order_acquire)) {
        out = g_info[dev];
    } else {
        // only a successful query is kept; a failed one is retried next call
        std::lock_guard<std::mutex> lock(g_info_mutex);
        if (!g_info_ready[dev].load(std::memory_order_relaxed)) {
            out = query_device(dev);
            if (out.err == hipSuccess) {
                g_info[dev] = out;
                g_info_ready[dev].store(true, std::memory_order_release);
            }
        } else {
            out = g_info[dev];
        }
    }
    if (out.err != hipSuccess)
        return fail(CSA_ERR_DEVICE, "cannot query device %d: %s", dev, hipGetErrorString(out.err));
    return CSA_OK;
}

csa_status device_lds_limit(size_t need, const char *what)
{
    DeviceInfo d;
    csa_status st = current_device(d);
    if (st != CSA_OK)
        return st;
    if (need > (size_t)d.lds)
        return fail(CSA_ERR_UNSUPPORTED, "%s needs %zu bytes of LDS per workgroup, device allows %d", what, need,
                    d.lds);
    return CSA_OK;
}

csa_status launched(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(CSA_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

// Top-k over rows of length up to W: the workgroup-per-row kernel for long
// rows when its LDS fits, else one wave per row.  When only the in-LDS part
// of the workgroup kernel fits (large k), it runs first and one wave per row
// then takes the rows it could not.
csa_status launch_topk_rows(csa::KernelArgs &a, hipStream_t s)
{
    DeviceInfo d;
    csa_status st = current_device(d);
    if (st != CSA_OK)
        return st;
    const int lim = d.lds;
    size_t block_lds = csa::topk_block_lds_bytes(a.cap, a.top_k, a.W);
    a.redo = 0;
    if (a.W >= csa::kTopkBlockMinLen && block_lds <= (size_t)lim)
        return launched(csa::launch_topk_block(a, block_lds, s), "top-k");
    size_t lds = csa::topk_lds_bytes(a.cap);
    if (lds > (size_t)lim)
        return fail(CSA_ERR_UNSUPPORTED, "top-k needs %zu bytes of LDS per workgroup, device allows %d", lds, lim);
    const size_t fast_lds = csa::topk_block_fast_only_lds_bytes(a.top_k, a.W);
    if (fast_lds != 0 && fast_lds <= (size_t)lim) {
        a.redo = 1;
        st = launched(csa::launch_topk_block(a, fast_lds, s), "top-k");
        if (st != CSA_OK)
            return st;
    }
    return launched(csa::launch_topk(a, lds, s), "top-k");
}

size_t select_workspace(const csa_index_problem *p, const Checked &c)
{
    if (c.plan != CSA_PLAN_SPLIT_ROWS)
        return 0;
    return (size_t)c.rows * (size_t)p->W * sizeof(float);
}

// Checks shared by the backward entry points.  The plan field is not used by
// the backward, so it is read as AUTO.
csa_status check_backward(const csa_index_problem *p, Checked &c, csa_index_problem &pa)
{
    if (!p)
        return fail(CSA_ERR_INVALID_ARG, "problem descriptor is NULL");
    pa = *p;
    pa.plan = CSA_PLAN_AUTO;
    csa_status st = check_problem(&pa, c);
    if (st != CSA_OK)
        return st;
    const int rpw = 4 / c.HB;
    const int64_t chunks = ((int64_t)pa.S + csa::kBwdChunkRows - 1) / csa::kBwdChunkRows;
    const int64_t jtiles = ((int64_t)pa.W + csa::kBwdKeyTile - 1) / csa::kBwdKeyTile;
    const int64_t rows_blocks = (int64_t)pa.B * (((int64_t)pa.S + rpw - 1) / rpw);
    const int64_t key_blocks = (int64_t)pa.B * 8 * ((chunks + 7) / 8) * jtiles;
    const int64_t red_blocks = ((int64_t)pa.B * pa.W * pa.D / 4 + 255) / 256;
    if (rows_blocks > 0x7FFFFFFF || key_blocks > 0x7FFFFFFF || red_blocks > 0x7FFFFFFF)
        return fail(CSA_ERR_UNSUPPORTED, "problem too large for one backward launch");
    // the workspace size (partials + sign words) must fit in size_t
    const unsigned __int128 part = (unsigned __int128)pa.B * chunks * pa.W * pa.D * 4;
    const unsigned __int128 sign = (unsigned __int128)pa.B * pa.S * (((int64_t)pa.W + 31) / 32) * pa.H * 4;
    if (part + sign + 256 > (unsigned __int128)SIZE_MAX / 2)
        return fail(CSA_ERR_UNSUPPORTED, "backward workspace too large");
    return CSA_OK;
}

// Fixed device scratch of csa_index_select_noalloc: one copy per GPU, held
// until the process ends.  Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol); each device's
// address comes from hipGetSymbolAddress, taken once with that device
// current.
constexpr size_t kNoAllocScratchBytes = CSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
std::atomic<bool> g_scratch_ready[kMaxDevices];
void *g_scratch_ptr[kMaxDevices]; // written once, under the mutex, before its flag is set

// Address of the current device's copy of `scratch`.
csa_status scratch_for_current_device(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(CSA_ERR_DEVICE, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(CSA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table holds", dev,
                    kMaxDevices);
    if (!g_scratch_ready[dev].load(std::memory_order_acquire)) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        if (!g_scratch_ready[dev].load(std::memory_order_relaxed)) {
            void *ptr = nullptr;
            hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || ptr == nullptr)
                return fail(CSA_ERR_DEVICE, "cannot resolve the scratch buffer on device %d: %s", dev,
                            hipGetErrorString(e));
            g_scratch_ptr[dev] = ptr;
            g_scratch_ready[dev].store(true, std::memory_order_release);
        }
    }
    *out = g_scratch_ptr[dev];
    return CSA_OK;
}

} // namespace

extern "C" {

int32_t csa_index_abi_version(void) { return CSA_INDEX_ABI_VERSION; }

const char *csa_status_string(csa_status s)
{
    // read as an int: a C caller may pass any value, and loading an enum
    // outside its enumerators' range is undefined in C++
    int v;
    std::memcpy(&v, &s, sizeof v);
    switch (v) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID_ARG: return "invalid argument";
    case CSA_ERR_UNSUPPORTED: return "unsupported shape or layout";
    case CSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA_ERR_DEVICE: return "device or launch error";
    default: return "unknown status";
    }
}

const char *csa_last_error(void) { return g_last_error.c_str(); }

int32_t csa_index_resolve_plan(const csa_index_problem *p)
{
    Checked c;
    if (check_problem(p, c) != CSA_OK)
        return -1;
    return c.plan;
}

csa_status csa_index_workspace_size(const csa_index_problem *p, int32_t top_k, size_t *bytes)
{
    if (!bytes)
        return fail(CSA_ERR_INVALID_ARG, "bytes is NULL");
    Checked c;
    csa_status st = check_problem(p, c);
    if (st != CSA_OK)
        return st;
    if (top_k < 1 || top_k > kMaxTopK)
        return fail(CSA_ERR_UNSUPPORTED, "top_k=%d outside [1, %d]", top_k, kMaxTopK);
    *bytes = select_workspace(p, c);
    return ok();
}

csa_status csa_index_topk_workspace_size(int64_t rows, int32_t W, int32_t top_k, size_t *bytes)
{
    if (!bytes)
        return fail(CSA_ERR_INVALID_ARG, "bytes is NULL");
    if (rows < 0 || W < 0)
        return fail(CSA_ERR_INVALID_ARG, "negative size");
    if (top_k < 1 || top_k > kMaxTopK)
        return fail(CSA_ERR_UNSUPPORTED, "top_k=%d outside [1, %d]", top_k, kMaxTopK);
    *bytes = 0;
    return ok();
}

csa_status csa_index_score(const csa_index_problem *p, const void *q, const void *k, const void *w,
                           const csa_index_masks *masks, float *scores, void *stream)
{
    Checked c;
    csa_status st = check_problem(p, c);
    if (st != CSA_OK)
        return st;
    if ((st = check_inputs(p, c, q, k, w, masks)) != CSA_OK)
        return st;
    if (c.rows * p->W == 0)
        return ok();
    if (!scores || !aligned(scores, 4))
        return fail(CSA_ERR_INVALID_ARG, "scores must be a non-NULL, 4-byte aligned pointer");
    csa::KernelArgs a = make_args(p, c, q, k, w, masks);
    a.scores = scores;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (c.plan == CSA_PLAN_SPLIT_ROWS) {
        a.full_rows = 1;
        return launched(csa::launch_split(p->D, c.HB, a, s), "split score");
    }
    size_t lds = csa::rows_lds_bytes(p->D, c.HB, csa::kModeScores, 0);
    return launched(csa::launch_rows(p->D, c.HB, csa::kModeScores, a, lds, s), "row-tile score");
}

csa_status csa_index_topk(int64_t rows, int32_t W, int32_t top_k, const float *scores, int32_t *idx,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    (void)workspace;
    (void)workspace_bytes;
    if (rows < 0 || W < 0)
        return fail(CSA_ERR_INVALID_ARG, "negative size (rows=%lld W=%d)", (long long)rows, W);
    if (top_k < 1 || top_k > kMaxTopK)
        return fail(CSA_ERR_UNSUPPORTED, "top_k=%d outside [1, %d]", top_k, kMaxTopK);
    if (W > kMaxW)
        return fail(CSA_ERR_UNSUPPORTED, "W=%d above the supported maximum %d", W, kMaxW);
    if (rows == 0)
        return ok();
    if (rows > (int64_t)0x7FFFFFFF * csa::kTopkWaves)
        return fail(CSA_ERR_UNSUPPORTED, "too many rows for one launch");
    if (!idx || !aligned(idx, 4))
        return fail(CSA_ERR_INVALID_ARG, "idx must be a non-NULL, 4-byte aligned pointer");
    if (W > 0 && (!scores || !aligned(scores, 4)))
        return fail(CSA_ERR_INVALID_ARG, "scores must be a non-NULL, 4-byte aligned pointer");
    csa::KernelArgs a{};
    a.scores = const_cast<float *>(scores);
    a.idx = idx;
    a.rows = rows;
    a.W = W;
    a.S = 1;
    a.m = 1;
    a.top_k = top_k;
    a.cap = csa::topk_capacity(top_k);
    return launch_topk_rows(a, static_cast<hipStream_t>(stream));
}

csa_status csa_index_select(const csa_index_problem *p, const void *q, const void *k, const void *w,
                            const csa_index_masks *masks, int32_t top_k, int32_t *idx, float *scores,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    Checked c;
    csa_status st = check_problem(p, c);
    if (st != CSA_OK)
        return st;
    if ((st = check_inputs(p, c, q, k, w, masks)) != CSA_OK)
        return st;
    if (top_k < 1 || top_k > kMaxTopK)
        return fail(CSA_ERR_UNSUPPORTED, "top_k=%d outside [1, %d]", top_k, kMaxTopK);
    if (c.rows == 0)
        return ok();
    if (!idx || !aligned(idx, 4))
        return fail(CSA_ERR_INVALID_ARG, "idx must be a non-NULL, 4-byte aligned pointer");
    if (scores && !aligned(scores, 4))
        return fail(CSA_ERR_INVALID_ARG, "scores must be 4-byte aligned");
    csa::KernelArgs a = make_args(p, c, q, k, w, masks);
    a.idx = idx;
    a.top_k = top_k;
    a.cap = csa::topk_capacity(top_k);
    hipStream_t s = static_cast<hipStream_t>(stream);

    if (c.plan == CSA_PLAN_SPLIT_ROWS) {
        float *buf = scores;
        if (!buf) {
            size_t need = select_workspace(p, c);
            if (need > 0 && (!workspace || workspace_bytes < need))
                return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                            workspace ? workspace_bytes : (size_t)0);
            if (!aligned(workspace, 256))
                return fail(CSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
            buf = static_cast<float *>(workspace);
        }
        a.scores = buf;
        a.full_rows = scores ? 1 : 0;
        if (p->W > 0) {
            // without a score output only the visible prefixes are needed:
            // few rows take the balanced split, others the chunked one
            DeviceInfo dinfo;
            if ((st = current_device(dinfo)) != CSA_OK)
                return st;
            const int cus = dinfo.cus;
            hipError_t e;
            // the balanced kernel's tile prefix is 32-bit
            const int64_t tiles_bound = c.rows * (((int64_t)p->W + csa::kTileEntries - 1) / csa::kTileEntries);
            if (!scores && c.rows <= csa::kStreamRows && tiles_bound < 0x7FFFFFFF)
                e = csa::launch_stream(p->D, c.HB, a, cus * csa::kStreamBlocksPerCU, s);
            else
                e = csa::launch_split(p->D, c.HB, a, s);
            if (e != hipSuccess)
                return launched(e, "split score");
        }
        a.limit_rows = 1;
        return launch_topk_rows(a, s);
    }

    const int mode = csa::kModeSelect | (scores ? csa::kModeScores : 0);
    a.cap = csa::rows_topk_capacity(top_k, c.HB);
    size_t lds = csa::rows_lds_bytes(p->D, c.HB, mode, a.cap);
    if ((st = device_lds_limit(lds, "row-tile select")) != CSA_OK)
        return st;
    a.scores = scores;
    return launched(csa::launch_rows(p->D, c.HB, mode, a, lds, s), "row-tile select");
}

csa_status csa_index_select_noalloc(const csa_index_problem *p, const void *q, const void *k, const void *w,
                                    const csa_index_masks *masks, int32_t top_k, int32_t *idx, float *scores,
                                    void *stream)
{
    Checked c;
    csa_status st = check_problem(p, c);
    if (st != CSA_OK)
        return st;
    if (top_k < 1 || top_k > kMaxTopK)
        return fail(CSA_ERR_UNSUPPORTED, "top_k=%d outside [1, %d]", top_k, kMaxTopK);
    // the workspace csa_index_select would take (none with a score output)
    const size_t need = scores ? 0 : select_workspace(p, c);
    if (need > kNoAllocScratchBytes)
        return fail(CSA_ERR_WORKSPACE,
                    "this problem needs %zu bytes of workspace, above the %zu-byte scratch of the "
                    "no-allocation entry point (use csa_index_select with a workspace)",
                    need, kNoAllocScratchBytes);
    if (need == 0)
        return csa_index_select(p, q, k, w, masks, top_k, idx, scores, nullptr, 0, stream);
    void *ws = nullptr;
    if ((st = scratch_for_current_device(&ws)) != CSA_OK)
        return st;
    return csa_index_select(p, q, k, w, masks, top_k, idx, scores, ws, kNoAllocScratchBytes, stream);
}

csa_status csa_index_kl_loss(const csa_index_problem *p, const void *q, const void *k, const void *w,
                             const csa_index_masks *masks, const float *target, float *kl, float *grad,
                             void *stream)
{
    if (!p)
        return fail(CSA_ERR_INVALID_ARG, "problem descriptor is NULL");
    // the plan field is not used: the loss runs on the row-tile kernel (any W)
    csa_index_problem pa = *p;
    pa.plan = CSA_PLAN_AUTO;
    Checked c;
    csa_status st = check_problem(&pa, c);
    if (st != CSA_OK)
        return st;
    if ((st = check_inputs(&pa, c, q, k, w, masks)) != CSA_OK)
        return st;
    if (c.rows == 0)
        return ok();
    if (c.rows > 0x7FFFFFFF)
        return fail(CSA_ERR_UNSUPPORTED, "too many rows for one launch");
    if (!kl || !aligned(kl, 4))
        return fail(CSA_ERR_INVALID_ARG, "kl must be a non-NULL, 4-byte aligned pointer");
    if (pa.W > 0 && (!target || !aligned(target, 4)))
        return fail(CSA_ERR_INVALID_ARG, "target must be a non-NULL, 4-byte aligned pointer");
    if (grad && !aligned(grad, 4))
        return fail(CSA_ERR_INVALID_ARG, "grad must be 4-byte aligned");
    csa::KernelArgs a = make_args(&pa, c, q, k, w, masks);
    a.target = target;
    a.kl = kl;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!grad) {
        const size_t lds = csa::rows_lds_bytes(pa.D, c.HB, csa::kModeKL, 0);
        if ((st = device_lds_limit(lds, "row-tile loss")) != CSA_OK)
            return st;
        return launched(csa::launch_rows(pa.D, c.HB, csa::kModeKL, a, lds, s), "row-tile loss");
    }
    // scores into the gradient buffer, then the loss and its gradient in place
    if ((st = csa_index_score(&pa, q, k, w, masks, grad, stream)) != CSA_OK)
        return st;
    a.scores = grad;
    return launched(csa::launch_kl_grad(a, s), "loss gradient");
}

csa_status csa_index_backward_workspace_size(const csa_index_problem *p, size_t *bytes)
{
    if (!bytes)
        return fail(CSA_ERR_INVALID_ARG, "bytes is NULL");
    Checked c;
    csa_index_problem pa;
    csa_status st = check_backward(p, c, pa);
    if (st != CSA_OK)
        return st;
    *bytes = csa::bwd_workspace_bytes(pa.B, pa.S, pa.W, pa.D, pa.H);
    return ok();
}

csa_status csa_index_score_backward(const csa_index_problem *p, const void *q, const void *k, const void *w,
                                    const csa_index_masks *masks, const float *grad, float *dq, float *dk,
                                    float *dw, void *workspace, size_t workspace_bytes, void *stream)
{
    Checked c;
    csa_index_problem pa;
    csa_status st = check_backward(p, c, pa);
    if (st != CSA_OK)
        return st;
    if ((st = check_inputs(&pa, c, q, k, w, masks)) != CSA_OK)
        return st;
    const int64_t nq = c.rows * pa.H, nk = (int64_t)pa.B * pa.W;
    if (nq > 0 && (!dq || !dw || !aligned(dq, 4) || !aligned(dw, 4)))
        return fail(CSA_ERR_INVALID_ARG, "dq and dw must be non-NULL, 4-byte aligned pointers");
    if (nk > 0 && (!dk || !aligned(dk, 16)))
        return fail(CSA_ERR_INVALID_ARG, "dk must be a non-NULL, 16-byte aligned pointer");
    if (c.rows * pa.W > 0 && (!grad || !aligned(grad, 4)))
        return fail(CSA_ERR_INVALID_ARG, "grad must be a non-NULL, 4-byte aligned pointer");
    const size_t need = csa::bwd_workspace_bytes(pa.B, pa.S, pa.W, pa.D, pa.H);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned(workspace, 256))
            return fail(CSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    }
    csa::BwdArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.w = static_cast<const uint16_t *>(w);
    if (masks) {
        a.q_offset = masks->q_offset;
        a.q_seg = masks->q_seg;
        a.k_seg = masks->k_seg;
    }
    a.g = grad;
    a.dq = dq;
    a.dk = dk;
    a.dw = dw;
    a.part = static_cast<float *>(workspace);
    if (need > 0)
        a.sign = reinterpret_cast<uint32_t *>(static_cast<unsigned char *>(workspace) +
                                              csa::bwd_sign_offset(pa.B, pa.S, pa.W, pa.D));
    a.q_sb = pa.q_sb;
    a.q_sh = pa.q_sh;
    a.q_ss = pa.q_ss;
    a.k_sb = pa.k_sb;
    a.k_sw = pa.k_sw;
    a.w_sb = pa.w_sb;
    a.w_ss = pa.w_ss;
    a.B = pa.B;
    a.S = pa.S;
    a.H = pa.H;
    a.D = pa.D;
    a.W = pa.W;
    a.m = pa.compress_rate;
    a.scale = pa.scale;
    a.n_chunks = (int)(((int64_t)pa.S + csa::kBwdChunkRows - 1) / csa::kBwdChunkRows);
    a.n_jtiles = (int)(((int64_t)pa.W + csa::kBwdKeyTile - 1) / csa::kBwdKeyTile);
    a.n_blk = (int)(((int64_t)pa.W + 31) / 32);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = csa::launch_bwd_rows(pa.D, c.HB, a, s);
    if (e != hipSuccess)
        return launched(e, "backward dq/dw");
    e = csa::launch_bwd_keys(pa.D, c.HB, a, s);
    if (e != hipSuccess)
        return launched(e, "backward dk partials");
    return launched(csa::launch_bwd_reduce(a, s), "backward dk reduction");
}

} // extern "C"
