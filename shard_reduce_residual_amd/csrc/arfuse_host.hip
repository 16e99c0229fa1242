// arfuse_host.hip -- the C ABI of libarfuse: argument validation, launch geometry and
// dispatch to the instantiated fused kernel, plus the two utility entry points (the
// quantiser's conversion alone, and a streaming copy for the HBM ceiling).
//
// Every argument is validated before the first HIP call. The only device queries are
// hipGetDevice, the compute-unit count and LDS size (cached per device), and, for calls
// whose rows are claimed from a counter, the stream's device and capture status.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "arfuse.h"
#include "arfuse_table.hpp"

namespace {

using arf::held_launch_fn;
using arf::launch_fn;

bool in_menu_c(int c) { return c == 1 || c == 2 || c == 4 || c == 8; }
bool in_menu_w(int w) { return w == 4 || w == 8 || w == 16; }

int pow2_at_least(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}
int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];   // 0 = not queried yet
std::atomic<int> g_lds_bytes[kMaxDevices];  // LDS bytes a workgroup may use; 0 = not queried
std::atomic<int> g_path{0}, g_waves{0}, g_chunks{0};

struct Plan {
    int path;      // 1 row per wavefront, 2 row per workgroup, 3 held rows, 4 row per
                   // workgroup with rows claimed in start order
    int waves;     // wavefronts per workgroup
    int chunks;    // 16-byte chunks per lane
    uint32_t grid; // workgroups
    int held;      // held-row kernel: rows per workgroup and phase
    uint32_t lds;  // dynamic LDS bytes per workgroup (held rows; the occupancy cap of path 4)
    int64_t claim_static;   // path 4: workgroups that keep the row of their index
    uint32_t claim_count;   // path 4: workgroups that claim a row (a multiple of 8 * split)
    int claim_split;        // path 4: counters the claims are spread over (1, 2 or 4)
};

struct DeviceInfo {
    int cus;       // compute units
    int lds;       // LDS bytes one workgroup may allocate
    int index;     // device ordinal (-1 when the caller gave the CU count)
};

// ---- row-claim counters -------------------------------------------------------------------
//
// Path 4 hands rows to workgroups from up to kMaxSplit device counters that every launch
// returns to 0. The counters are this file-scope array, on every device the library runs
// on; nothing is allocated. A slot holds one stream's counters, one 256-byte line each (so
// no two share a cache line or an atomic unit's queue). A slot belongs to one stream: calls
// on one stream run one after another, so they may share it, and calls on different
// streams, which may overlap, never do. Calls that must not claim (see claim_counter) take
// the same kernel with rows by workgroup index.
constexpr int kClaimSlots = 256;
constexpr int kMaxSplit = 4;
constexpr int kSlotWords = 64 * kMaxSplit;
static __device__ __align__(256) uint32_t scratch[kClaimSlots * kSlotWords];

struct ClaimTable {
    std::mutex mu;
    uint32_t* base[kMaxDevices] = {};    // device address of `scratch` (hipGetSymbolAddress)
    bool unusable[kMaxDevices] = {};     // the symbol address could not be obtained
    uintptr_t owner[kMaxDevices][kClaimSlots] = {};   // stream handle + 1; 0 = free
};
ClaimTable g_claims;

// The counters of `stream` on device `dev`, or NULL when the call must not claim rows:
//  * the stream is being captured: a captured graph may be replayed on another stream;
//  * the per-thread default stream: one handle stands for a different stream per thread;
//  * the stream belongs to another device than the current one;
//  * every slot of the device belongs to another stream, or the symbol's address could not
//    be obtained.
// A slot, once given to a stream handle, stays with it for the life of the process.
uint32_t* claim_counter(int dev, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (dev < 0 || dev >= kMaxDevices || st == hipStreamPerThread) return nullptr;
    if (st) {
        hipDevice_t sd = -1;
        if (hipStreamGetDevice(st, &sd) != hipSuccess || sd != dev) return nullptr;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_claims.mu);
    if (!g_claims.base[dev]) {
        if (g_claims.unusable[dev]) return nullptr;
        void* ptr = nullptr;   // the current device is `dev`: its copy of the array
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            g_claims.unusable[dev] = true;
            return nullptr;
        }
        g_claims.base[dev] = static_cast<uint32_t*>(ptr);
    }
    const uintptr_t key = (uintptr_t)stream + 1;
    for (int i = 0; i < kClaimSlots; ++i) {
        uintptr_t& o = g_claims.owner[dev][i];
        if (o == 0) o = key;
        if (o == key) return g_claims.base[dev] + (size_t)i * kSlotWords;
    }
    return nullptr;
}

// Held-row kernel geometry: 4 or 8 wavefronts, one workgroup per compute unit, each
// holding up to as many rows as its LDS takes (the row's residual plus 12 bytes per
// wavefront for the partial sums of squares and the per-token maxima). Rows are spread
// evenly over the phases. Returns false when the row does not fit the kernel's menu (more
// than 8 chunks per lane with 4 wavefronts or 4 with 8, or a single row larger than the
// LDS).
// LDS per workgroup assumed by arf_get_plan when the caller gives a CU count instead of
// querying a device: gfx950's 160 KiB.
constexpr int kPlanLdsBytes = 160 * 1024;
bool held_plan(int64_t rows, int32_t hidden, const DeviceInfo& dev, int waves, int chunks,
               Plan* pl) {
    const int hc = hidden / 8;
    if (chunks == 0) chunks = pow2_at_least(div_up(hc, waves * 64));
    if (chunks > (waves == 8 ? 4 : 8) || waves * 64 * chunks < hc) return false;
    // per held row: the residual plus each wavefront's sum of squares and maximum
    const int64_t per_row = (int64_t)hidden * 2 + waves * 12;
    const int64_t kmax = dev.lds / per_row;
    if (kmax < 1) return false;
    const int64_t grid = rows < dev.cus ? rows : dev.cus;
    const int64_t phases = div_up(rows, grid * kmax);
    const int64_t k = div_up(rows, grid * phases);
    pl->path = 3;
    pl->waves = waves;
    pl->chunks = chunks;
    pl->grid = (uint32_t)grid;
    pl->held = (int)k;
    pl->lds = (uint32_t)(k * per_row);
    return true;
}


// Launch geometry: the hidden/8 chunks of a row are spread over the lanes that own it.
// Fitted to sweeps on MI355X (256 CUs) over hidden 1024..16384, 128..8192 tokens, 2 and 8
// bf16 shards and 4 fp32 shards, and checked on other shapes (hidden 1536..12288, 4 and 16
// bf16, 8 fp16 and 2 fp32 shards), where it stays within 1.1% of the best menu entry on
// geometric mean:
//  * one row per wavefront (4 rows per workgroup) for short rows: rows of <= 64 chunks
//    always, rows of <= 128 chunks from 2 rows per compute unit, rows of <= 256 chunks from
//    8 rows per compute unit;
//  * otherwise one row per workgroup:
//    - few rows (< 2 per compute unit) of more than 256 chunks: 8 wavefronts per row, so
//      that each row exposes more parallel loads; rows of up to 256 chunks fill no more
//      than 4 wavefronts' lanes, and 4 wavefronts measured 6-22% faster than 8 there
//      (graph replay of 1-511 rows, hidden 512-2048, 2 and 8 shards; one row per
//      wavefront 13-35% faster still for 64-chunk rows);
//    - otherwise 4 wavefronts with up to 8 chunks per lane, so that several rows share a
//      compute unit;
//    - rows too wide for 8 chunks per lane use 16 wavefronts.
//  * held rows (path 3) where that measured faster (sweep of 175 shapes, bit-identical
//    outputs, and 150 more, see held_eight and held_wins): 4096 <= hidden <= 8192, no
//    quantised copy, from 3 rows per compute unit up to what one batch per workgroup
//    holds; for fp32 partials beyond 4 shards, shards x chunks per lane <= 48; with a
//    per-tensor fp8 copy, most of that range (see held_wins). There HBM sees the whole launch's reads,
//    then its writes: 2-10% faster (3% for 4 fp32 shards of 2048 x 7168). With more
//    shards, other row sizes, several batches, or the per-token scale's extra pass over the
//    held rows, it was slower than one row per workgroup.
//  * rows claimed in start order (path 4, the same kernel as path 2) where a sweep of 32
//    shapes (1-16 shards, hidden 4096-16384, 1024-16384 tokens, bf16 and fp32 partials)
//    measured it faster: 4 wavefronts per row, and either at least 16 rows per compute unit
//    with at least 128 KiB of traffic per row, or at least 8 rows per compute unit with at
//    least 256 KiB per row: 1-8% faster (8 shards of 8192 x 16384 with per-token fp8:
//    512-528 -> 481-487 us). With fewer rows per compute unit there is little drift to
//    correct. Two workgroups per compute unit (an LDS reservation caps them) measured
//    faster than three with claims on every shape; the first two workgroups per compute
//    unit keep their own row, so the launch's first wave of workgroups does not queue on
//    the counter at once.
//  * one counter serves about 50 claims per microsecond; shorter rows claim faster than
//    that, so their claims are spread over 2 or 4 counters (a sweep of 22 shapes, 2-16
//    shards, hidden 2048-16384, against rows by index, row per wavefront and one counter):
//    rows of 128-256 KiB take 2 counters (up to 1.6% faster than one; at 256 KiB and more
//    one counter stays as fast); from 32 rows per compute unit, rows of 96-128 KiB take 2
//    counters and 2 workgroups per compute unit (4 x 16384 x 8192: -3%), rows of 32-96 KiB
//    with at least 256 chunks take 4 counters and 4 workgroups per compute unit (8 x 16384
//    x 4096: -6%; 16 x 16384 x 2048: -9% against one row per wavefront). Rows of 28 KiB
//    and launches of 16 rows per compute unit gained nothing and keep their plans.
// The held-row kernel with 8 wavefronts (half the chunks per lane, 2 wavefronts per SIMD)
// exists for 16-bit partials, for every shard count, without a quantised copy and in the
// general form. Without a copy, with 1-4 shards it measured -7% to +1.6% against 4
// wavefronts over the held region (better on balance), and 1% slower for fp32 partials.
// With 5-16 shards it opens the held region to them: against the plan's rows by index or
// claims it was 2-12% faster on 38 of 40 shapes (5, 6, 8, 12, 16 shards, hidden 4096-8192,
// 6-16 rows per CU; 16 x 3072 x 4096: 83.9 -> 73.6 us), level on 8 x 1536 x 4096 and 3%
// slower on 16 x 2048 x 8192. With a per-tensor copy see held_wins; with a per-token copy
// (forced held rows only) it was faster than 4 wavefronts on 19 of 24 shapes.
bool held_eight(int pdt, int32_t hidden) {
    return pdt != ARF_F32 && pow2_at_least(div_up(hidden / 8, 8 * 64)) <= 4;
}

bool held_wins(int64_t tokens, int32_t hidden, int n, int quant, int pdt, const DeviceInfo& dev,
               Plan* pl) {
    bool eight = held_eight(pdt, hidden);
    // From 3 rows per CU (3-5 rows per CU, 2-16 shards, hidden 4096-8192: 1-12% faster
    // than rows by index on all 36 shapes, 16-bit and fp32) up to as many as one batch
    // holds (17-19 rows per CU of hidden 4096: up to 9% faster, level for 2 bf16 shards).
    // Hidden 2048 was 23-38% slower than one row per wavefront.
    const bool held_region = hidden >= 4096 && hidden <= 8192 && tokens >= 3LL * dev.cus;
    if (!held_region) return false;
    if (quant == arf::kQuantTensor) {
        // A per-tensor fp8 copy takes the general form, where it measured faster than rows
        // by index (7 interleaved repetitions each; one shard was not faster throughout):
        //  - fp32 partials, 4 wavefronts, 2-8 shards: hidden 6144-8192 from 3 rows per CU
        //    (16 of 16 shapes 0.3-9.4% faster) and hidden 4096 from 8 rows per CU (12 of
        //    12, 1.1-9.3%); hidden 5120 (-2.3% to +5.9%) and 4096 at 3-4 rows per CU
        //    (-4.3% to +1.9%) were mixed;
        //  - 16-bit partials, 2-4 shards, hidden 6144-8192, from 6 rows per CU: 4 wavefronts
        //    (10 of 10 shapes 2.8-9.1% faster; 4 x 2048 x 7168: 39.9 -> 36.5 us; 8
        //    wavefronts were -0.5% to +4.9% against 4 there);
        //  - 16-bit partials otherwise 8 wavefronts: 2-4 shards at hidden 6144-8192 below 6
        //    rows per CU (11 of 11, 0.3-13%), below hidden 6144 (9 of 9, 2.3-6.8%), 5-8 shards
        //    (18 of 18, 0.4-7.9%) and 9-16 shards from 8 rows per CU (9 of 10, 2.3-9.2%; one
        //    +0.6%); 9-16 shards at 3-4 rows per CU were mixed (-3.7% to +5.2%).
        if (n < 2 || tokens < (pdt != ARF_F32 && n > 8 ? 8LL : 3LL) * dev.cus) return false;
        if (pdt == ARF_F32) {
            if (n > 8 || !(hidden >= 6144 || (hidden == 4096 && tokens >= 8LL * dev.cus)))
                return false;
        } else if (n <= 4 && hidden >= 6144 && tokens >= 6LL * dev.cus) {
            eight = false;
        }
    } else if (quant == arf::kQuantMx) {
        // An MXFP4 copy takes the general form over the region without a copy, 9-16 16-bit
        // shards from 8 rows per CU: 19 of 20 shapes 0.1-7.0% faster than rows by index,
        // one +0.4% (1-16 shards, hidden 4096-8192, 3-19 rows per CU); 16 x 1024 x 8192
        // was 3.5% slower.
        if (pdt != ARF_F32 && n > 8 && tokens < 8LL * dev.cus) return false;
    } else if (quant != arf::kQuantNone) {
        return false;
    }
    Plan h;
    if (!held_plan(tokens, hidden, dev, eight ? 8 : 4, 0, &h)) return false;
    // fp32 partials beyond 4 shards: the 4-wavefront form, where shards x chunks per lane
    // <= 48 (without a copy, 5-16 shards, 6-16 rows per CU: 0.5-10% faster than rows by
    // index or claims on 34 of 40 shapes; 16 shards x 4 chunks ran out of registers, 16-23%
    // slower)
    if (!eight && n > 4 && (h.chunks > 4 || n * h.chunks > 48)) return false;
    if ((int64_t)h.grid * h.held < tokens) return false;   // more than one batch
    *pl = h;
    return true;
}

// The claim rules of the plan (path 4), from the launch-geometry notes above: the counters
// the claims are spread over (0: rows by index) and the workgroups per compute unit.
struct ClaimRule {
    int split;
    int per_cu;
};
ClaimRule claim_rule(int64_t tokens, int64_t row_bytes, int hc, int waves, const DeviceInfo& dev) {
    if (waves != 4) return {0, 0};
    if ((tokens >= 16LL * dev.cus && row_bytes >= 128 * 1024) ||
        (tokens >= 8LL * dev.cus && row_bytes >= 256 * 1024))
        return {row_bytes >= 256 * 1024 ? 1 : 2, 2};
    if (tokens >= 32LL * dev.cus && hc >= 256 && row_bytes >= 32 * 1024) {
        if (row_bytes >= 96 * 1024) return {2, 2};
        return {4, 4};
    }
    return {0, 0};
}

// Forced claims (tests): the split of the plan's rules for the row size.
ClaimRule forced_claim_rule(int64_t row_bytes) {
    return row_bytes < 96 * 1024    ? ClaimRule{4, 4}
           : row_bytes < 256 * 1024 ? ClaimRule{2, 2}
                                    : ClaimRule{1, 2};
}

// Static LDS of the fused kernel (per-wavefront partial sums and maxima, the claimed row),
// left free beside the path-4 reservation so that exactly two workgroups fit a compute unit.
constexpr int kStaticLdsSlack = 2048;

// row_bytes: HBM traffic of one row (partials, residual, outputs), for the claim rule.
arf_status make_plan(int64_t tokens, int32_t hidden, int n, int pdt, int quant,
                     int64_t row_bytes, const DeviceInfo& dev, bool reduce_only, Plan* pl) {
    const int hc = hidden / 8;
    const int num_cus = dev.cus;
    int path = g_path.load(), waves = g_waves.load(), chunks = g_chunks.load();
    pl->held = 0;
    pl->lds = 0;
    pl->claim_static = 0;
    pl->claim_count = 0;
    pl->claim_split = 0;
    if (path == 3) {
        // the held-row kernel has no reduce-only form: such calls take the default plan.
        // Without a forced wave count, the plan's: 8 where that form exists and fits.
        if (!reduce_only) {
            const bool eight = held_eight(pdt, hidden);
            if (waves == 0 && eight && held_plan(tokens, hidden, dev, 8, chunks, pl)) return ARF_OK;
            if (waves == 8 && !eight) return ARF_ERR_VALUE;
            return held_plan(tokens, hidden, dev, waves ? waves : 4, chunks, pl) ? ARF_OK
                                                                                : ARF_ERR_VALUE;
        }
        path = waves = chunks = 0;
    }
    if (path == 0 && !reduce_only && held_wins(tokens, hidden, n, quant, pdt, dev, pl))
        return ARF_OK;
    const bool forced_claims = path == 4;
    ClaimRule rule = forced_claims ? forced_claim_rule(row_bytes) : ClaimRule{0, 0};
    if (path == 0) {
        waves = chunks = 0;
        const bool many_rows = tokens >= 2LL * num_cus;
        rule = claim_rule(tokens, row_bytes, hc, 4, dev);
        if (rule.split == 0 && (hc <= 64 || (hc <= 128 && many_rows) ||
                                (hc <= 256 && tokens >= 8LL * num_cus))) {
            path = 1;
        } else {
            path = 2;
            waves = many_rows || hc <= 256 ? 4 : 8;
            if (hc > waves * 64 * 8) waves = 16;
            chunks = pow2_at_least(div_up(hc, waves * 64));
            if (waves != 4) rule = ClaimRule{0, 0};
        }
    }
    if (path == 1) {
        waves = 4;
        if (chunks == 0) chunks = pow2_at_least(div_up(hc, 64));
        if (chunks > 8 || 64 * chunks < hc) return ARF_ERR_VALUE;
        pl->grid = (uint32_t)((tokens + 3) / 4);
    } else {
        if (waves == 0 && chunks == 0) {   // forced path, free geometry: as the plan's
            waves = hc > 4 * 64 * 8 ? 16 : 4;
            chunks = pow2_at_least(div_up(hc, waves * 64));
        } else if (waves == 0) {
            for (waves = 4; waves < 16 && waves * 64 * chunks < hc; waves *= 2) {}
        } else if (chunks == 0) {
            chunks = pow2_at_least(div_up(hc, waves * 64));
        }
        if (chunks > 8 || waves * 64 * chunks < hc) return ARF_ERR_VALUE;
        pl->grid = (uint32_t)tokens;
        path = 2;
        if (rule.split > 0) {
            // forced (tests): every row is claimed; planned: the first per_cu workgroups
            // per compute unit keep their row. One claiming workgroup per 16 rows (at
            // least 64) beyond the rows is the slack that lets a faster XCD take more
            // rows; the claimants are a multiple of 8 * split, so that every counter has
            // as many as the others.
            const int64_t first =
                forced_claims ? 0 : std::min<int64_t>(tokens, (int64_t)rule.per_cu * num_cus);
            const int64_t unit = 8LL * rule.split;
            const int64_t count =
                div_up(tokens - first + std::max<int64_t>(64, tokens / 16), unit) * unit;
            const int64_t grid = first + count;
            if (grid * 64 * waves <= (int64_t)UINT32_MAX) {   // one dispatch, else path 2
                path = 4;
                pl->claim_static = first;
                pl->claim_count = (uint32_t)count;
                pl->claim_split = rule.split;
                pl->grid = (uint32_t)grid;
                pl->lds = (uint32_t)((dev.lds - kStaticLdsSlack) / rule.per_cu);
            }
        }
    }
    pl->path = path;
    pl->waves = waves;
    pl->chunks = chunks;
    return ARF_OK;
}

held_launch_fn lookup_held(int pdt, int adt, int n, int c, bool quant, int waves) {
#define ARF_BY_RANGE(PD, AD)                                                 \
    if (n <= 4) return arf::held_##PD##_##AD##_n01_04(n, c, quant, waves);   \
    if (n <= 8) return arf::held_##PD##_##AD##_n05_08(n, c, quant, waves);   \
    if (n <= 12) return arf::held_##PD##_##AD##_n09_12(n, c, quant, waves);  \
    return arf::held_##PD##_##AD##_n13_16(n, c, quant, waves);
    if (adt == ARF_BF16) {
        if (pdt == ARF_F32) { ARF_BY_RANGE(f32, bf16) }
        ARF_BY_RANGE(bf16, bf16)
    }
    if (pdt == ARF_F32) { ARF_BY_RANGE(f32, f16) }
    ARF_BY_RANGE(f16, f16)
#undef ARF_BY_RANGE
}

launch_fn lookup(int pdt, int adt, int n, const Plan& pl) {
    const bool rpw = pl.path == 1;
    const int w = pl.waves, c = pl.chunks;
#define ARF_BY_RANGE(PD, AD)                                                   \
    if (n <= 4) return arf::lookup_##PD##_##AD##_n01_04(n, rpw, w, c);         \
    if (n <= 8) return arf::lookup_##PD##_##AD##_n05_08(n, rpw, w, c);         \
    if (n <= 12) return arf::lookup_##PD##_##AD##_n09_12(n, rpw, w, c);        \
    return arf::lookup_##PD##_##AD##_n13_16(n, rpw, w, c);
    if (adt == ARF_BF16) {
        if (pdt == ARF_F32) { ARF_BY_RANGE(f32, bf16) }
        ARF_BY_RANGE(bf16, bf16)
    }
    if (pdt == ARF_F32) { ARF_BY_RANGE(f32, f16) }
    ARF_BY_RANGE(f16, f16)
#undef ARF_BY_RANGE
}

arf_status device_info(DeviceInfo* info) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ARF_ERR_HIP;
    if (dev < kMaxDevices) {
        const int c = g_cu_count[dev].load(std::memory_order_relaxed);
        const int l = g_lds_bytes[dev].load(std::memory_order_relaxed);
        if (c > 0 && l > 0) {
            *info = DeviceInfo{c, l, dev};
            return ARF_OK;
        }
    }
    int c = 0, l = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        c <= 0)
        return ARF_ERR_HIP;
    if (hipDeviceGetAttribute(&l, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        l <= 0)
        return ARF_ERR_HIP;
    if (dev < kMaxDevices) {
        g_cu_count[dev].store(c, std::memory_order_relaxed);
        g_lds_bytes[dev].store(l, std::memory_order_relaxed);
    }
    *info = DeviceInfo{c, l, dev};
    return ARF_OK;
}

arf_status device_cus(int* cus) {
    DeviceInfo info;
    const arf_status st = device_info(&info);
    if (st == ARF_OK) *cus = info.cus;
    return st;
}

struct Range {
    uintptr_t b, e;
};
Range span(const void* p, int64_t bytes) {
    return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)(bytes > 0 ? bytes : 0)};
}
bool overlap(Range a, Range b) { return a.b < b.e && b.b < a.e; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

struct Call {
    const void* partials;
    int32_t n;
    int64_t tokens;
    int64_t row_begin;
    int64_t row_count;   // < 0: through the last row
    int32_t hidden;
    int32_t pdt, adt;
    int32_t acc;         // ARF_ACC_*
    const void* residual_in;
    void* residual_out;  // the reduced values in reduce-only mode
    const void* gamma;
    float eps;
    void* norm_out;
    uint8_t* quant_out;
    int32_t quant;       // arf::QuantMode
    const float* scale_in;
    void* scale_out;
    bool reduce_only;
};

// Order: sizes, types, mode and eps first; then the row range. An empty range is then a
// complete call, so its pointers may be NULL (zero-size tensors often have no address);
// otherwise pointers, alignment and overlaps (over the buffers' full [tokens] extents).
arf_status validate(Call& c) {
    if (c.n < 1 || c.n > ARF_MAX_SHARDS || c.tokens < 0 || c.tokens > INT32_MAX ||
        c.hidden <= 0 || c.hidden % 8 != 0 || c.hidden > ARF_MAX_HIDDEN)
        return ARF_ERR_SHAPE;
    if (c.adt != ARF_BF16 && c.adt != ARF_F16) return ARF_ERR_DTYPE;
    if (c.pdt != c.adt && c.pdt != ARF_F32) return ARF_ERR_DTYPE;
    if (c.acc != ARF_ACC_F32 && c.acc != ARF_ACC_PARTIAL) return ARF_ERR_VALUE;
    if (!(c.eps >= 0.0f) || std::isinf(c.eps)) return ARF_ERR_VALUE;
    if (c.row_begin < 0 || c.row_begin > c.tokens) return ARF_ERR_SHAPE;
    if (c.row_count < 0) c.row_count = c.tokens - c.row_begin;
    if (c.row_count > c.tokens - c.row_begin) return ARF_ERR_SHAPE;
    if (c.row_count == 0) return ARF_OK;
    if (!c.partials) return ARF_ERR_NULL;
    if (c.reduce_only) {
        if (!c.residual_out) return ARF_ERR_NULL;
    } else {
        if (!c.residual_in || !c.gamma) return ARF_ERR_NULL;
        if (c.quant == arf::kQuantTensor && (!c.quant_out || !c.scale_in)) return ARF_ERR_NULL;
        if ((c.quant == arf::kQuantToken || c.quant == arf::kQuantMx) &&
            (!c.quant_out || !c.scale_out))
            return ARF_ERR_NULL;
        if (c.quant == arf::kQuantMx && c.hidden % 32 != 0) return ARF_ERR_SHAPE;
        if (c.quant == arf::kQuantNone && !c.residual_out && !c.norm_out)
            return ARF_ERR_NO_OUTPUT;
    }
    const void* t16[] = {c.partials, c.residual_in, c.residual_out, c.gamma, c.norm_out,
                         c.quant_out};
    for (const void* p : t16)
        if (p && !aligned(p, 16)) return ARF_ERR_ALIGN;
    if ((c.quant == arf::kQuantTensor && !aligned(c.scale_in, 4)) ||
        (c.quant == arf::kQuantToken && !aligned(c.scale_out, 4)))
        return ARF_ERR_ALIGN;

    const int64_t th = c.tokens * (int64_t)c.hidden;
    const int64_t sp = c.pdt == ARF_F32 ? 4 : 2;
    Range in_part = span(c.partials, (int64_t)c.n * th * sp);
    Range in_res = c.residual_in ? span(c.residual_in, th * 2) : Range{0, 0};
    Range in_gam = c.gamma ? span(c.gamma, (int64_t)c.hidden * 2) : Range{0, 0};
    Range in_sc = c.quant == arf::kQuantTensor ? span(c.scale_in, 4) : Range{0, 0};
    Range outs[4] = {
        c.residual_out ? span(c.residual_out, th * 2) : Range{0, 0},
        c.norm_out ? span(c.norm_out, th * 2) : Range{0, 0},
        c.quant == arf::kQuantMx      ? span(c.quant_out, th / 2)
        : c.quant != arf::kQuantNone ? span(c.quant_out, th)
                                     : Range{0, 0},
        c.quant == arf::kQuantToken ? span(c.scale_out, c.tokens * 4)
        : c.quant == arf::kQuantMx  ? span(c.scale_out, th / 32)
                                    : Range{0, 0},
    };
    for (int i = 0; i < 4; ++i) {
        const Range o = outs[i];
        if (o.b == o.e) continue;
        if (overlap(o, in_part) || overlap(o, in_gam) || overlap(o, in_sc)) return ARF_ERR_ALIAS;
        const bool in_place = i == 0 && c.residual_out == c.residual_in;
        if (!in_place && overlap(o, in_res)) return ARF_ERR_ALIAS;
        for (int k = i + 1; k < 4; ++k)
            if (outs[k].b != outs[k].e && overlap(o, outs[k])) return ARF_ERR_ALIAS;
    }
    return ARF_OK;
}

arf_status run(Call c, void* stream) {
    arf_status st = validate(c);
    if (st != ARF_OK || c.row_count == 0) return st;
    DeviceInfo dev;
    if ((st = device_info(&dev)) != ARF_OK) return st;
    const int64_t sp = c.pdt == ARF_F32 ? 4 : 2;
    const int64_t qbytes = c.quant == arf::kQuantMx     ? c.hidden / 2 + c.hidden / 32
                           : c.quant != arf::kQuantNone ? c.hidden
                                                        : 0;
    const int64_t row_bytes = (int64_t)c.n * c.hidden * sp + 2LL * c.hidden * 3 + qbytes;
    Plan pl;
    if ((st = make_plan(c.row_count, c.hidden, c.n, c.pdt, c.quant, row_bytes, dev,
                        c.reduce_only, &pl)) != ARF_OK)
        return st;
    uint32_t* counter = pl.path == 4 ? claim_counter(dev.index, stream) : nullptr;
    if (pl.path == 4 && !counter) {   // the same kernel with rows by workgroup index
        pl.path = 2;
        pl.grid = (uint32_t)c.row_count;
        pl.lds = 0;
    }
    launch_fn fn = nullptr;
    held_launch_fn hfn = nullptr;
    if (pl.path == 3)
        hfn = lookup_held(c.pdt, c.adt, c.n, pl.chunks, c.quant != arf::kQuantNone, pl.waves);
    else fn = lookup(c.pdt, c.adt, c.n, pl);
    if (!fn && !hfn) return ARF_ERR_VALUE;
    arf::Params p;
    p.partials = c.partials;
    p.residual_in = c.reduce_only ? nullptr : c.residual_in;
    p.residual_out = c.residual_out;
    p.gamma = c.gamma;
    p.norm_out = c.reduce_only ? nullptr : c.norm_out;
    p.quant_out = c.quant_out;
    p.scale_in = c.scale_in;
    p.scale_out = c.scale_out;
    p.tokens = c.tokens;
    p.row_begin = c.row_begin;
    p.row_end = c.row_begin + c.row_count;
    p.hidden = c.hidden;
    p.n_shards = c.n;
    p.eps = c.eps;
    p.quant_mode = c.reduce_only ? arf::kQuantNone : c.quant;
    p.acc_partial = c.acc == ARF_ACC_PARTIAL;
    p.reduce_only = c.reduce_only;
    p.held_rows = pl.held;
    p.claim = nullptr;
    p.claim_static = 0;
    p.claim_count = 0;
    p.claim_shift = 0;
    if (hfn)   // at most one workgroup per compute unit, looping over its rows
        return hfn(p, pl.grid, pl.lds, (hipStream_t)stream) == hipSuccess ? ARF_OK : ARF_ERR_HIP;
    if (pl.path == 4) {   // one dispatch (the plan checked its size)
        p.claim = counter;
        p.claim_static = pl.claim_static;
        p.claim_count = pl.claim_count;
        p.claim_shift = pl.claim_split == 4 ? 2u : pl.claim_split == 2 ? 1u : 0u;
        return fn(p, pl.grid, pl.lds, (hipStream_t)stream) == hipSuccess ? ARF_OK : ARF_ERR_HIP;
    }
    // One dispatch covers at most 2^32 - 1 work-items: a grid that would exceed that is
    // split into consecutive row ranges, one kernel each, enqueued in row order.
    const int64_t threads = pl.path == 1 ? 256 : 64LL * pl.waves;
    const int64_t rows_per_wg = pl.path == 1 ? 4 : 1;
    const int64_t max_rows = ((int64_t)UINT32_MAX / threads) * rows_per_wg;
    const int64_t end = c.row_begin + c.row_count;
    for (int64_t b = c.row_begin; b < end; b += max_rows) {
        p.row_begin = b;
        p.row_end = end - b < max_rows ? end : b + max_rows;
        const uint32_t grid = (uint32_t)((p.row_end - b + rows_per_wg - 1) / rows_per_wg);
        if (fn(p, grid, 0, (hipStream_t)stream) != hipSuccess) return ARF_ERR_HIP;
    }
    return ARF_OK;
}

// ---- utility kernels -----------------------------------------------------------------------

__global__ __launch_bounds__(256) void e4m3_encode_kernel(const float* __restrict__ in,
                                                          uint8_t* __restrict__ out,
                                                          int64_t n) {
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n;
         i += (int64_t)gridDim.x * 256 * 4) {
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = i + k < n ? in[i + k] : 0.0f;
        const uint32_t w = arf::e4m3x4(v[0], v[1], v[2], v[3]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (i + k < n) out[i + k] = (uint8_t)(w >> (8 * k));
    }
}

// One E2M1 code per byte (the low nibble), through the MXFP4 store's conversion.
__global__ __launch_bounds__(256) void e2m1_encode_kernel(const float* __restrict__ in,
                                                          uint8_t* __restrict__ out,
                                                          int64_t n) {
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n;
         i += (int64_t)gridDim.x * 256 * 4) {
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = i + k < n ? in[i + k] : 0.0f;
        const uint32_t w = arf::e2m1_pack4(v[0], v[1], v[2], v[3]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (i + k < n) out[i + k] = (uint8_t)((w >> (4 * k)) & 0xFu);
    }
}

// Contiguous spans of 256 lanes x 8 x 16 bytes per workgroup iteration, through a buffer
// resource per span (the fused kernel's load/store forms, non-temporal).
constexpr int kCopyUnroll = 8;
constexpr int64_t kCopySpan = 256 * kCopyUnroll * 16;

__global__ __launch_bounds__(256) void stream_copy_kernel(char* __restrict__ dst,
                                                          const char* __restrict__ src,
                                                          int64_t bytes) {
    for (int64_t s = (int64_t)blockIdx.x * kCopySpan; s < bytes;
         s += (int64_t)gridDim.x * kCopySpan) {
        const int64_t left = bytes - s;
        const uint32_t n = (uint32_t)(left < kCopySpan ? left : kCopySpan);
        const auto rs = arf::make_rsrc(src + s, n);
        const auto rd = arf::make_rsrc(dst + s, n);
        arf::u32x4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(
                rs, (uint32_t)(u * 256 + threadIdx.x) * 16u, 0, arf::kAuxStream);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(
                v[u], rd, (uint32_t)(u * 256 + threadIdx.x) * 16u, 0, arf::kAuxStream);
    }
}

// Streaming probe with a given read/write mix: unit u reads its share of src (16 KiB
// spans, non-temporal), then writes its share of dst with a value that depends on what it
// read, so each unit's writes follow its reads as in the fused kernel's rows.
constexpr int kMixUnroll = 4;
constexpr int64_t kMixSpan = 256 * kMixUnroll * 16;

__global__ __launch_bounds__(256) void stream_mix_kernel(char* __restrict__ dst,
                                                         int64_t write_bytes,
                                                         const char* __restrict__ src,
                                                         int64_t read_bytes, int64_t units) {
    const int64_t sr = (read_bytes + kMixSpan - 1) / kMixSpan;
    const int64_t sw = (write_bytes + kMixSpan - 1) / kMixSpan;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        uint32_t acc = (uint32_t)u;
        for (int64_t k = u * sr / units; k < (u + 1) * sr / units; ++k) {
            const int64_t left = read_bytes - k * kMixSpan;
            const auto rs = arf::make_rsrc(src + k * kMixSpan,
                                           (uint32_t)(left < kMixSpan ? left : kMixSpan));
            arf::u32x4 v[kMixUnroll];
#pragma unroll
            for (int i = 0; i < kMixUnroll; ++i)
                v[i] = __builtin_amdgcn_raw_buffer_load_b128(
                    rs, (uint32_t)(i * 256 + threadIdx.x) * 16u, 0, arf::kAuxStream);
#pragma unroll
            for (int i = 0; i < kMixUnroll; ++i) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
        }
        // keep the loads live when nothing is written (an empty statement, no instruction)
        __asm__ volatile("" : : "v"(acc));
        const arf::u32x4 w = {acc, acc + 1u, acc + 2u, acc + 3u};
        for (int64_t k = u * sw / units; k < (u + 1) * sw / units; ++k) {
            const int64_t left = write_bytes - k * kMixSpan;
            const auto rd = arf::make_rsrc(dst + k * kMixSpan,
                                           (uint32_t)(left < kMixSpan ? left : kMixSpan));
#pragma unroll
            for (int i = 0; i < kMixUnroll; ++i)
                __builtin_amdgcn_raw_buffer_store_b128(
                    w, rd, (uint32_t)(i * 256 + threadIdx.x) * 16u, 0, arf::kAuxStream);
        }
    }
}

}  // namespace

extern "C" {

arf_status arf_reduce_add_rmsnorm(const void* partials, int32_t n_shards, int64_t tokens,
                                  int32_t hidden, int32_t partial_dtype, int32_t act_dtype,
                                  const void* residual_in, void* residual_out,
                                  const void* gamma, float eps, void* norm_out,
                                  void* stream) {
    Call c{partials, n_shards, tokens, 0, -1, hidden, partial_dtype, act_dtype, ARF_ACC_F32,
           residual_in, residual_out, gamma, eps, norm_out, nullptr, arf::kQuantNone,
           nullptr, nullptr, false};
    return run(c, stream);
}

arf_status arf_reduce_add_rmsnorm_quant(const void* partials, int32_t n_shards,
                                        int64_t tokens, int32_t hidden,
                                        int32_t partial_dtype, int32_t act_dtype,
                                        const void* residual_in, void* residual_out,
                                        const void* gamma, float eps, void* norm_out,
                                        uint8_t* quant_out, int32_t mode,
                                        const float* scale_in, float* scale_out,
                                        void* stream) {
    int32_t q;
    if (mode == ARF_QUANT_PER_TENSOR) q = arf::kQuantTensor;
    else if (mode == ARF_QUANT_PER_TOKEN) q = arf::kQuantToken;
    else return ARF_ERR_VALUE;
    Call c{partials, n_shards, tokens, 0, -1, hidden, partial_dtype, act_dtype, ARF_ACC_F32,
           residual_in, residual_out, gamma, eps, norm_out, quant_out, q,
           q == arf::kQuantTensor ? scale_in : nullptr,
           q == arf::kQuantToken ? scale_out : nullptr, false};
    return run(c, stream);
}

arf_status arf_fused_epilogue(const arf_params* a, void* stream) {
    if (!a) return ARF_ERR_NULL;
    if (a->struct_size != sizeof(arf_params)) return ARF_ERR_VALUE;
    int32_t q = arf::kQuantNone;
    if (a->quant_out) {
        if (a->quant_mode == ARF_QUANT_PER_TENSOR) q = arf::kQuantTensor;
        else if (a->quant_mode == ARF_QUANT_PER_TOKEN) q = arf::kQuantToken;
        else if (a->quant_mode == ARF_QUANT_MXFP4) q = arf::kQuantMx;
        else return ARF_ERR_VALUE;
    }
    Call c{a->partials, a->n_shards, a->tokens, a->row_begin, a->row_count, a->hidden,
           a->partial_dtype, a->act_dtype, a->accumulate, a->residual_in, a->residual_out,
           a->gamma, a->eps, a->norm_out, q != arf::kQuantNone ? a->quant_out : nullptr, q,
           q == arf::kQuantTensor ? a->scale_in : nullptr,
           (q == arf::kQuantToken || q == arf::kQuantMx) ? a->scale_out : nullptr, false};
    return run(c, stream);
}

arf_status arf_reduce_rows(const void* partials, int32_t n_shards, int64_t tokens,
                           int64_t row_begin, int64_t row_count, int32_t hidden,
                           int32_t partial_dtype, int32_t act_dtype, int32_t accumulate,
                           void* sums_out, void* stream) {
    Call c{partials, n_shards, tokens, row_begin, row_count, hidden, partial_dtype,
           act_dtype, accumulate, nullptr, sums_out, nullptr, 0.0f, nullptr, nullptr,
           arf::kQuantNone, nullptr, nullptr, true};
    return run(c, stream);
}

const char* arf_status_string(int32_t s) {
    switch (s) {
        case ARF_OK: return "ARF_OK";
        case ARF_ERR_NULL: return "ARF_ERR_NULL: a required pointer is NULL";
        case ARF_ERR_SHAPE: return "ARF_ERR_SHAPE: n_shards, tokens or hidden out of range";
        case ARF_ERR_DTYPE: return "ARF_ERR_DTYPE: unsupported element type combination";
        case ARF_ERR_ALIGN: return "ARF_ERR_ALIGN: misaligned pointer";
        case ARF_ERR_ALIAS: return "ARF_ERR_ALIAS: an output overlaps another buffer";
        case ARF_ERR_NO_OUTPUT: return "ARF_ERR_NO_OUTPUT: no output requested";
        case ARF_ERR_VALUE: return "ARF_ERR_VALUE: bad eps, mode or geometry override";
        case ARF_ERR_HIP: return "ARF_ERR_HIP: no usable device or launch failure";
        default: return "unknown arf_status";
    }
}

int32_t arf_version(void) { return ARF_VERSION; }

arf_status arf_get_plan_quant(int32_t n_shards, int64_t tokens, int32_t hidden,
                              int32_t partial_dtype, int32_t quant_mode, int32_t num_cus,
                              int32_t* out) {
    if (!out) return ARF_ERR_NULL;
    if (n_shards < 1 || n_shards > ARF_MAX_SHARDS || tokens < 0 || tokens > INT32_MAX ||
        hidden <= 0 || hidden % 8 != 0 || hidden > ARF_MAX_HIDDEN)
        return ARF_ERR_SHAPE;
    if (partial_dtype != ARF_BF16 && partial_dtype != ARF_F16 && partial_dtype != ARF_F32)
        return ARF_ERR_DTYPE;
    int32_t q;
    if (quant_mode == ARF_QUANT_NONE) q = arf::kQuantNone;
    else if (quant_mode == ARF_QUANT_PER_TENSOR) q = arf::kQuantTensor;
    else if (quant_mode == ARF_QUANT_PER_TOKEN) q = arf::kQuantToken;
    else if (quant_mode == ARF_QUANT_MXFP4) q = arf::kQuantMx;
    else return ARF_ERR_VALUE;
    if (q == arf::kQuantMx && hidden % 32 != 0) return ARF_ERR_SHAPE;
    DeviceInfo dev{num_cus, kPlanLdsBytes, -1};
    if (num_cus <= 0) {
        arf_status st = device_info(&dev);
        if (st != ARF_OK) return st;
    }
    const int64_t qbytes = q == arf::kQuantMx     ? hidden / 2 + hidden / 32
                           : q != arf::kQuantNone ? hidden
                                                  : 0;
    const int64_t row_bytes = (int64_t)n_shards * hidden * (partial_dtype == ARF_F32 ? 4 : 2) +
                              2LL * hidden * 3 + qbytes;
    Plan pl;
    arf_status st = make_plan(tokens, hidden, n_shards, partial_dtype, q, row_bytes, dev, false,
                              &pl);
    if (st != ARF_OK) return st;
    out[0] = pl.path;
    out[1] = pl.waves;
    out[2] = pl.chunks;
    out[3] = (int32_t)pl.grid;
    return ARF_OK;
}

arf_status arf_get_plan(int32_t n_shards, int64_t tokens, int32_t hidden,
                        int32_t partial_dtype, int32_t num_cus, int32_t* out) {
    return arf_get_plan_quant(n_shards, tokens, hidden, partial_dtype, ARF_QUANT_NONE, num_cus,
                              out);
}

arf_status arf_set_path_override(int32_t path, int32_t waves_per_block,
                                 int32_t chunks_per_lane) {
    if (path < 0 || path > 4) return ARF_ERR_VALUE;
    if (path == 0 && (waves_per_block || chunks_per_lane)) return ARF_ERR_VALUE;
    if (path == 1 && waves_per_block && waves_per_block != 4) return ARF_ERR_VALUE;
    if (path == 3 && waves_per_block && waves_per_block != 4 && waves_per_block != 8)
        return ARF_ERR_VALUE;
    if ((path == 2 || path == 4) && waves_per_block && !in_menu_w(waves_per_block))
        return ARF_ERR_VALUE;
    if (chunks_per_lane && !in_menu_c(chunks_per_lane)) return ARF_ERR_VALUE;
    g_path.store(path);
    g_waves.store(path >= 2 ? waves_per_block : 0);   // path 1 uses 4
    g_chunks.store(chunks_per_lane);
    return ARF_OK;
}

arf_status arf_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream) {
    if (n < 0) return ARF_ERR_SHAPE;
    if (n == 0) return ARF_OK;
    if (!in || !out) return ARF_ERR_NULL;
    if (!aligned(in, 4)) return ARF_ERR_ALIGN;
    if (overlap(span(in, n * 4), span(out, n))) return ARF_ERR_ALIAS;
    // 1024 elements per workgroup and pass; the kernel loops when the grid is capped at
    // one dispatch's 2^32 - 1 work-items
    const int64_t blocks = std::min<int64_t>((n + 1023) / 1024, (int64_t)UINT32_MAX / 256);
    void* args[] = {&in, &out, &n};
    return hipLaunchKernel(reinterpret_cast<const void*>(&e4m3_encode_kernel),
                           dim3((uint32_t)blocks), dim3(256), args, 0,
                           (hipStream_t)stream) == hipSuccess
               ? ARF_OK
               : ARF_ERR_HIP;
}

arf_status arf_e2m1_encode(const float* in, uint8_t* out, int64_t n, void* stream) {
    if (n < 0) return ARF_ERR_SHAPE;
    if (n == 0) return ARF_OK;
    if (!in || !out) return ARF_ERR_NULL;
    if (!aligned(in, 4)) return ARF_ERR_ALIGN;
    if (overlap(span(in, n * 4), span(out, n))) return ARF_ERR_ALIAS;
    const int64_t blocks = std::min<int64_t>((n + 1023) / 1024, (int64_t)UINT32_MAX / 256);
    void* args[] = {&in, &out, &n};
    return hipLaunchKernel(reinterpret_cast<const void*>(&e2m1_encode_kernel),
                           dim3((uint32_t)blocks), dim3(256), args, 0,
                           (hipStream_t)stream) == hipSuccess
               ? ARF_OK
               : ARF_ERR_HIP;
}

arf_status arf_stream_copy(void* dst, const void* src, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16 != 0) return ARF_ERR_SHAPE;
    if (bytes == 0) return ARF_OK;
    if (!dst || !src) return ARF_ERR_NULL;
    if (!aligned(dst, 16) || !aligned(src, 16)) return ARF_ERR_ALIGN;
    if (overlap(span(dst, bytes), span(src, bytes))) return ARF_ERR_ALIAS;
    int cus = 0;
    arf_status st = device_cus(&cus);
    if (st != ARF_OK) return st;
    const int64_t spans = (bytes + kCopySpan - 1) / kCopySpan;
    const int64_t cap = (int64_t)cus * 16;
    const uint32_t grid = (uint32_t)(spans < cap ? spans : cap);
    char* d = (char*)dst;
    const char* s = (const char*)src;
    void* args[] = {&d, &s, &bytes};
    return hipLaunchKernel(reinterpret_cast<const void*>(&stream_copy_kernel), dim3(grid),
                           dim3(256), args, 0, (hipStream_t)stream) == hipSuccess
               ? ARF_OK
               : ARF_ERR_HIP;
}

arf_status arf_stream_mix(void* dst, int64_t write_bytes, const void* src, int64_t read_bytes,
                          int64_t units, void* stream) {
    if (read_bytes < 0 || write_bytes < 0 || read_bytes % 16 != 0 || write_bytes % 16 != 0)
        return ARF_ERR_SHAPE;
    if (read_bytes == 0 && write_bytes == 0) return ARF_OK;
    if ((read_bytes && !src) || (write_bytes && !dst)) return ARF_ERR_NULL;
    if ((read_bytes && !aligned(src, 16)) || (write_bytes && !aligned(dst, 16)))
        return ARF_ERR_ALIGN;
    if (read_bytes && write_bytes && overlap(span(dst, write_bytes), span(src, read_bytes)))
        return ARF_ERR_ALIAS;
    const int64_t sr = (read_bytes + kMixSpan - 1) / kMixSpan;
    const int64_t sw = (write_bytes + kMixSpan - 1) / kMixSpan;
    if (units <= 0) units = sr && sw ? (sr < sw ? sr : sw) : (sr ? sr : sw);
    if (units > INT32_MAX) return ARF_ERR_SHAPE;
    int cus = 0;
    arf_status st = device_cus(&cus);
    if (st != ARF_OK) return st;
    // one workgroup per unit, capped at one dispatch's 2^32 - 1 work-items (the kernel
    // loops over the units)
    const uint32_t grid = (uint32_t)std::min<int64_t>(units, (int64_t)UINT32_MAX / 256);
    char* d = (char*)dst;
    const char* sp = (const char*)src;
    void* args[] = {&d, &write_bytes, &sp, &read_bytes, &units};
    return hipLaunchKernel(reinterpret_cast<const void*>(&stream_mix_kernel), dim3(grid),
                           dim3(256), args, 0, (hipStream_t)stream) == hipSuccess
               ? ARF_OK
               : ARF_ERR_HIP;
}

}  // extern "C"
