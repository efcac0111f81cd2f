// ep_api.hip -- host side of the C ABI declared in include/ep.h: argument
// validation, the per-context workspace, launch geometry and status words.
// Every step of the hot path runs in the kernels of ep_kernels.hip.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "ep.h"
#include "ep_internal.h"

struct ep_ctx {
    ep_config cfg;
    int device;
    int num_tiles;
    int keys;  // E + R
    void *ws;
    size_t ws_bytes;
    uint32_t *counters;
    uint32_t *status;  // where the kernels OR their status bits (the workspace's status word)
    uint64_t *tile_state;
    uint64_t *bp;
    uint32_t *rank_ready;
    uint32_t spin_limit;
    bool debug;
    int cu_count;
    int fused_per_cu[2][2][2];  // [deduplicated][k > 8][fp8]: fused-kernel blocks one CU holds (-1: not asked)
    int cu_budget;             // compute units the caller's stream may use (ep_set_cu_budget; 0 = all)
};

namespace {

// Waves a token-major launch aims for. Dispatch (write-heavy, one read of x
// per token) keeps a token's passes in one wave; combine (k gathered rows per
// pass) splits every token into one wave per 1024-channel pass, which keeps
// more independent row loads in flight.
constexpr int kDispatchTargetWaves = 2048;  // ~8 waves per CU on 256 CUs
constexpr int kCombineTargetWaves = 1 << 30;  // i.e. one pass per wave
// The backward's gradient dispatch (rows from the handle, BF16, no layout in
// the same grid) also runs one pass per wave: on MI355X with rotated buffers
// 106.9 vs 109.6 us at 4096 tokens x 7168 and 424.8 vs 439.9 us at 16384,
// with the row loader's full set of 16 loads per wave (a build that issued
// only the wave's 2 took 110 us). (The fused grids must stay within the
// resident blocks; the low-latency kernel and the forward dispatch gain
// nothing from more waves.)
constexpr int kBackwardTargetWaves = 1 << 30;
constexpr int kFusedMaxTiles = 16;
constexpr uint32_t kDefaultSpinLimit = 1u << 20;  // polls of a bounded wait before EP_ST_TIMEOUT             // layout tiles up to which one grid does layout + dispatch
constexpr int kMaxPassPerWave = 8;   // must match ep_kernels.hip

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int validate_config(const ep_config *c) {
    if (!c) return EP_ERR_ARG;
    if (c->reserved != 0) return EP_ERR_ARG;
    if (c->num_ranks < 1 || c->num_ranks > ep::kMaxRanks) return EP_ERR_ARG;
    if (c->num_tokens < 0 || c->num_tokens > (1 << 24) || c->num_tokens % c->num_ranks) return EP_ERR_ARG;
    if (c->num_topk < 1 || c->num_topk > ep::kMaxTopk) return EP_ERR_ARG;
    if (c->num_experts < 1 || c->num_experts > ep::kMaxExperts || c->num_experts % c->num_ranks)
        return EP_ERR_ARG;
    if (c->hidden < 8 || c->hidden > 65536 || c->hidden % 8) return EP_ERR_ARG;
    if (c->cap_rows < 0 || (int64_t)c->num_ranks * c->cap_rows >= ((int64_t)1 << 31)) return EP_ERR_ARG;
    return EP_OK;
}

int num_tiles_of(const ep_config &c) {
    const int n = (c.num_tokens + ep::kLayoutTile - 1) / ep::kLayoutTile;
    return n > 0 ? n : 1;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// workspace: counters | tile states | boundary prefixes (epoch-tagged) |
// rank-ready flags (one per layout block of a fused launch)
struct WorkspaceLayout {
    size_t state, bp, rank_ready, total;
};

WorkspaceLayout workspace_layout(const ep_config &c) {
    const size_t keys = (size_t)c.num_experts + c.num_ranks;
    const size_t tiles = (size_t)num_tiles_of(c);
    const size_t blocks = tiles > (size_t)ep::kLayoutReplicas ? tiles : (size_t)ep::kLayoutReplicas;
    WorkspaceLayout w;
    size_t off = round_up(ep::kNumCounters * sizeof(uint32_t), 256);
    w.state = off;
    off = round_up(off + tiles * keys * sizeof(uint64_t), 256);
    w.bp = off;
    off = round_up(off + ((size_t)c.num_ranks + 1) * keys * sizeof(uint64_t), 256);
    w.rank_ready = off;
    off = round_up(off + blocks * sizeof(uint32_t), 256);
    w.total = off;
    return w;
}

// Work split of a token-major kernel: waves_per_token waves share a token's
// rows, each taking passes_per_wave passes of 1024 channels.
struct Geometry {
    int npass, wpt, ppw, num_waves;
};

Geometry geometry(int T, int H, int target_waves) {
    Geometry g;
    g.npass = (H + 1023) / 1024;
    int w = T > 0 ? (int)(((int64_t)target_waves + T - 1) / T) : 1;
    const int minw = (g.npass + kMaxPassPerWave - 1) / kMaxPassPerWave;
    if (w < minw) w = minw;
    if (w > g.npass) w = g.npass;
    g.ppw = (g.npass + w - 1) / w;
    g.wpt = (g.npass + g.ppw - 1) / g.ppw;
    g.num_waves = T * g.wpt;
    return g;
}

int hip_fail(hipError_t e, const char *what) {
    if (e == hipSuccess) return EP_OK;
    std::fprintf(stderr, "libep: %s failed: %s\n", what, hipGetErrorString(e));
    return EP_ERR_HIP;
}

// The context's workspace lives on the device that was current at
// ep_create; a call made with another device current would hand its kernels
// that workspace. (EP_ERR_ARG: make the context's device current.)
int check_device(const ep_ctx *ctx) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return EP_ERR_HIP;
    return dev == ctx->device ? EP_OK : EP_ERR_ARG;
}

int check_handle(const ep_ctx *ctx, const ep_handle *h) {
    if (!h) return EP_ERR_ARG;
    if (h->num_tokens != ctx->cfg.num_tokens || h->num_topk != ctx->cfg.num_topk) return EP_ERR_ARG;
    if (!h->pos && ctx->cfg.num_tokens > 0) return EP_ERR_ARG;
    return EP_OK;
}

// compute units the context's launches may use (its budget, else the device's)
int usable_cus(const ep_ctx *ctx) {
    return ctx->cu_budget > 0 ? std::min(ctx->cu_budget, ctx->cu_count) : ctx->cu_count;
}

int combine_common(ep_ctx *ctx, const uint16_t *rows, const ep_handle *h, const float *w, void *out,
                   bool out_f32, ep_stream_t stream, const char *name) {
    if (!ctx) return EP_ERR_ARG;
    if (int r = check_device(ctx)) return r;
    if (int r = check_handle(ctx, h)) return r;
    const ep_config &c = ctx->cfg;
    if (c.num_tokens == 0) return EP_OK;
    if (!out || (!rows && c.cap_rows > 0)) return EP_ERR_ARG;
    if (!aligned(out, 16) || !aligned(rows, 16) || !aligned(h->pos, 4) || !aligned(w, 4)) return EP_ERR_ALIGN;
    const Geometry g = geometry(c.num_tokens, c.hidden, kCombineTargetWaves);
    ep::CombineArgs a;
    a.rows = rows;
    a.pos = h->pos;
    a.w = w;
    a.out = out;
    a.T = c.num_tokens;
    a.k = c.num_topk;
    a.H = c.hidden;
    a.num_rows = (int64_t)c.num_ranks * c.cap_rows;
    a.waves_per_token = g.wpt;
    a.passes_per_wave = g.ppw;
    a.npass = g.npass;
    a.counters = ctx->counters;
    a.status = ctx->status;
    if (ctx->debug)
        std::fprintf(stderr, "libep: %s T=%d k=%d H=%d waves=%d (%d/token, %d passes each)\n", name, a.T, a.k,
                     a.H, g.num_waves, g.wpt, g.ppw);
    // the residency cap is measured for a stream that has every CU
    const int cap_cus = ctx->cu_budget > 0 && ctx->cu_budget < ctx->cu_count ? 0 : ctx->cu_count;
    return hip_fail(ep::launch_combine(a, out_f32, false, g.num_waves, cap_cus, (hipStream_t)stream), name);
}

// The expert-side pre-reduction of deduplicated rows: the combine kernel over
// the received rows (see ep_prereduce in ep.h).
int prereduce_common(ep_ctx *ctx, const uint16_t *expert_out, const int32_t *recv_topk_idx,
                     const float *recv_topk_w, const int32_t *token_rows, void *out, bool out_f32,
                     ep_stream_t stream, const char *name) {
    if (!ctx) return EP_ERR_ARG;
    if (int r = check_device(ctx)) return r;
    const ep_config &c = ctx->cfg;
    const int64_t rows = (int64_t)c.num_ranks * c.cap_rows;
    if (rows == 0) return EP_OK;
    if (rows * c.num_topk >= ((int64_t)1 << 31)) return EP_ERR_ARG;  // per-(row, slot) outputs indexed by int
    if (!expert_out || !recv_topk_idx || !token_rows || !out) return EP_ERR_ARG;
    if (!aligned(expert_out, 16) || !aligned(out, 16) || !aligned(recv_topk_idx, 4) || !aligned(recv_topk_w, 4) ||
        !aligned(token_rows, 4))
        return EP_ERR_ALIGN;
    const Geometry g = geometry((int)rows, c.hidden, kCombineTargetWaves);
    ep::CombineArgs a;
    std::memset(&a, 0, sizeof a);
    a.rows = expert_out;
    a.pos = recv_topk_idx;
    a.w = recv_topk_w;
    a.out = out;
    a.T = (int)rows;
    a.k = c.num_topk;
    a.H = c.hidden;
    a.num_rows = rows * c.num_topk;
    a.token_rows = token_rows;
    a.cap_rows = c.cap_rows;
    a.waves_per_token = g.wpt;
    a.passes_per_wave = g.ppw;
    a.npass = g.npass;
    a.counters = ctx->counters;
    a.status = ctx->status;
    if (ctx->debug)
        std::fprintf(stderr, "libep: %s rows=%lld k=%d H=%d waves=%d\n", name, (long long)rows, a.k, a.H,
                     g.num_waves);
    return hip_fail(ep::launch_combine(a, out_f32, true, g.num_waves, 0, (hipStream_t)stream), name);
}

// log2(v) when v is a power of two, else -1
int log2_exact(int v) {
    if (v <= 0 || (v & (v - 1))) return -1;
    int s = 0;
    while ((1 << s) < v) ++s;
    return s;
}

// mode: 0 = rows from the handle (backward), 1 = per expert, 2 = per rank
int fill_dispatch(ep_ctx *ctx, const uint16_t *x, const int32_t *topk, const float *w, const ep_layout *L,
                  int mode, void *recv_x, float *recv_scales, float *recv_w, ep_handle *h, ep::DispatchArgs &a,
                  Geometry &g, int target_waves = kDispatchTargetWaves) {
    const ep_config &c = ctx->cfg;
    if (!x || (!recv_x && c.cap_rows > 0)) return EP_ERR_ARG;
    if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(h->pos, 4)) return EP_ERR_ALIGN;
    g = geometry(c.num_tokens, c.hidden, target_waves);
    std::memset(&a, 0, sizeof a);
    a.x = x;
    a.topk = topk;
    a.w = w;
    a.pos = h->pos;
    a.src_idx = h->src_idx;
    a.recv_w = (w && recv_w) ? recv_w : nullptr;
    a.recv_x = recv_x;
    a.recv_scales = recv_scales;
    if (mode != 0) {
        a.rank_in_expert = L->rank_in_expert;
        a.expert_off = L->expert_off;
        a.rank_in_rank = L->rank_in_rank;
    }
    a.T = c.num_tokens;
    a.k = c.num_topk;
    a.E = c.num_experts;
    a.epr = c.num_experts / c.num_ranks;
    a.epr_shift = log2_exact(a.epr);
    a.H = c.hidden;
    a.cap_rows = c.cap_rows;
    a.num_rows = (int64_t)c.num_ranks * c.cap_rows;
    a.waves_per_token = g.wpt;
    a.passes_per_wave = g.ppw;
    a.npass = g.npass;
    a.counters = ctx->counters;
    a.status = ctx->status;
    return EP_OK;
}

int dispatch_common(ep_ctx *ctx, const uint16_t *x, const int32_t *topk, const float *w, const ep_layout *L,
                    bool fp8, int mode, void *recv_x, float *recv_scales, float *recv_w, ep_handle *h,
                    ep_stream_t stream, const char *name, int32_t *recv_topk_idx = nullptr,
                    float *recv_topk_w = nullptr) {
    const ep_config &c = ctx->cfg;
    if (c.num_tokens == 0) return EP_OK;
    ep::DispatchArgs a;
    Geometry g;
    if (int r = fill_dispatch(ctx, x, topk, w, L, mode, recv_x, recv_scales, recv_w, h, a, g,
                              mode == 0 ? kBackwardTargetWaves : kDispatchTargetWaves))
        return r;
    a.recv_topk_idx = recv_topk_idx;
    a.recv_topk_w = (w && recv_topk_w) ? recv_topk_w : nullptr;
    if (ctx->debug)
        std::fprintf(stderr, "libep: %s T=%d k=%d H=%d fp8=%d waves=%d (%d/token, %d passes each)\n", name,
                     a.T, a.k, a.H, (int)fp8, g.num_waves, g.wpt, g.ppw);
    return hip_fail(ep::launch_dispatch(a, fp8, mode, g.num_waves, (hipStream_t)stream), name);
}

int fill_layout(ep_ctx *ctx, const int32_t *topk_idx, const ep_layout *L, ep::LayoutArgs &a) {
    if (!ctx || !L) return EP_ERR_ARG;
    if (int r = check_device(ctx)) return r;
    const ep_config &c = ctx->cfg;
    if (!L->cnt_se || !L->cnt_sd || !L->recv_cnt || !L->expert_off || !L->rank_rows || !L->src_expert_off)
        return EP_ERR_ARG;
    if (c.num_tokens > 0 && (!topk_idx || !L->rank_in_expert || !L->is_token_in_rank)) return EP_ERR_ARG;
    if (!aligned(topk_idx, 4) || !aligned(L->rank_in_expert, 16) || !aligned(L->is_token_in_rank, 16) ||
        !aligned(L->cnt_se, 4) || !aligned(L->cnt_sd, 4) || !aligned(L->recv_cnt, 4) ||
        !aligned(L->expert_off, 4) || !aligned(L->rank_rows, 4) || !aligned(L->src_expert_off, 4))
        return EP_ERR_ALIGN;
    std::memset(&a, 0, sizeof a);
    // the slot loads read a clamped row even with no tokens: then they read
    // the workspace (at least kMaxTopk ints) instead of a possibly null array
    a.topk = c.num_tokens > 0 ? topk_idx : reinterpret_cast<const int32_t *>(ctx->ws);
    a.T = c.num_tokens;
    a.k = c.num_topk;
    a.E = c.num_experts;
    a.R = c.num_ranks;
    a.epr = c.num_experts / c.num_ranks;
    a.epr_shift = log2_exact(a.epr);
    a.tpr = c.num_tokens / c.num_ranks;
    a.num_tiles = ctx->num_tiles;
    a.use_ticket = ctx->num_tiles > ep::kCoResidentTiles;
    a.cap_rows = c.cap_rows;
    a.rank_in_expert = L->rank_in_expert;
    a.itr = L->is_token_in_rank;
    a.cnt_se = L->cnt_se;
    a.cnt_sd = L->cnt_sd;
    a.recv_cnt = L->recv_cnt;
    a.expert_off = L->expert_off;
    a.rank_rows = L->rank_rows;
    a.src_expert_off = L->src_expert_off;
    a.tile_state = ctx->tile_state;
    a.bp = ctx->bp;
    a.rank_ready = ctx->rank_ready;
    a.counters = ctx->counters;
    a.status = ctx->status;
    a.spin_limit = ctx->spin_limit;
    // the deduplicated outputs: both or neither (no tokens: rank_in_rank is empty)
    if (L->rank_in_rank && !L->token_rows) return EP_ERR_ARG;
    if (L->token_rows && !L->rank_in_rank && c.num_tokens > 0) return EP_ERR_ARG;
    if (!aligned(L->rank_in_rank, 16) || !aligned(L->token_rows, 4)) return EP_ERR_ALIGN;
    a.rank_in_rank = L->rank_in_rank;
    a.token_rows = L->token_rows;
    return EP_OK;
}

// Shared checks of the forward dispatch arguments; sets the handle's config.
// The fused layout+dispatch grid, sized for the compute units the caller's
// stream may use (mode 1: per expert, 2: deduplicated per rank). Beyond
// kFusedMaxTiles tiles the layout and the dispatch run as two launches: the
// dispatch waves that fill the GPU would otherwise wait through a longer
// layout while their row loads crowd its memory round trips (measured on
// MI355X: 8192 tokens, 170 us as two launches against 212 us fused).
int launch_fused(ep_ctx *ctx, const ep::LayoutArgs &la, const ep::DispatchArgs &da, bool fp8, int mode,
                 int num_waves, ep_stream_t stream, const char *name) {
    const ep_config &c = ctx->cfg;
    if (ctx->num_tiles > kFusedMaxTiles) {
        if (int r = hip_fail(ep::launch_layout(la, (hipStream_t)stream), name)) return r;
        return hip_fail(ep::launch_dispatch(da, fp8, mode, num_waves, (hipStream_t)stream), name);
    }
    int &per_cu = ctx->fused_per_cu[mode == 2][c.num_topk > 8][fp8];
    if (per_cu < 0)
        per_cu = ep::layout_dispatch_blocks_per_cu(c.num_topk, fp8, mode,
                                                   ep::layout_lds_bytes(c.num_experts + c.num_ranks));
    const int cus = usable_cus(ctx);
    return hip_fail(ep::launch_layout_dispatch(la, da, fp8, mode, num_waves, cus * per_cu, (hipStream_t)stream),
                    name);
}

int check_forward_dispatch(ep_ctx *ctx, const int32_t *topk_idx, const float *topk_weights, const ep_layout *L,
                           int use_fp8, float *recv_scales, float *recv_w, ep_handle *handle) {
    if (!ctx || !L || !handle) return EP_ERR_ARG;
    if (int r = check_device(ctx)) return r;
    const ep_config &c = ctx->cfg;
    if (use_fp8 != 0 && use_fp8 != 1) return EP_ERR_ARG;
    if (use_fp8 && (c.hidden % 128 || (!recv_scales && c.cap_rows > 0))) return EP_ERR_ARG;
    if (!use_fp8 && recv_scales) return EP_ERR_ARG;
    if ((!handle->pos && c.num_tokens > 0) || (!handle->src_idx && c.cap_rows > 0)) return EP_ERR_ARG;
    if (c.num_tokens > 0 && (!topk_idx || !L->rank_in_expert || !L->expert_off)) return EP_ERR_ARG;
    if (!aligned(topk_idx, 4) || !aligned(topk_weights, 4) || !aligned(recv_w, 4) || !aligned(recv_scales, 4) ||
        !aligned(handle->src_idx, 4))
        return EP_ERR_ALIGN;
    handle->num_tokens = c.num_tokens;
    handle->num_topk = c.num_topk;
    return EP_OK;
}

int dispatch_with_layout(ep_ctx *ctx, const uint16_t *x, const int32_t *topk_idx, const float *topk_weights,
                         const ep_layout *L, int use_fp8, void *recv_x, float *recv_scales, float *recv_w,
                         ep_handle *handle, ep_stream_t stream);

// ---------------------------------------------------------------------------
// The workspace of ep_dispatch_with_layout_noalloc, for callers that cannot
// allocate: a static device array (each GPU the library runs on holds its
// own copy until the process ends). Zero at load, which is a valid workspace
// start (see ep_internal.h). Its host-side name is not a device address:
// host code uses only the address hipGetSymbolAddress returns for the
// current device, taken once per device.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)4 << 20;
constexpr int kMaxDevices = 64;
// Each part of the array has one fixed place whatever the call's sizes, so
// that a word always holds the same kind of value (a flag an epoch, a
// look-back state a tagged state): a call of one size never reads what a
// call of another size stored (its boundary prefixes, say) as a ready flag.
constexpr int kScratchMaxTiles = 4096;
constexpr size_t kScratchRankReady = 256;  // after the counters: [layout blocks] flags
constexpr size_t kScratchBp = kScratchRankReady + (size_t)kScratchMaxTiles * 4;  // [R+1][E+R] tagged prefixes
constexpr size_t kScratchStates =
    kScratchBp + ((size_t)(ep::kMaxRanks + 1) * (ep::kMaxExperts + ep::kMaxRanks) * 8 + 255) / 256 * 256;

// Whether a config's layout fits the static workspace: its tiles' flags and
// look-back states ([tiles][E+R] 8-byte words after the fixed parts).
bool fits_scratch(const ep_config &c) {
    const size_t tiles = (size_t)num_tiles_of(c), keys = (size_t)c.num_experts + c.num_ranks;
    return tiles <= (size_t)kScratchMaxTiles && tiles * keys * 8 <= kScratchBytes - kScratchStates;
}

struct ScratchDevice {
    void *ptr;                  // the array's address on this device (NULL until set up)
    int cu_count;
    int fused_per_cu[2][2][2];  // as ep_ctx::fused_per_cu
    uint32_t spin_limit;
    bool debug;
};

std::mutex g_scratch_mu;
ScratchDevice g_scratch_dev[kMaxDevices];

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// The static workspace on device `dev` (current), set up on its first use.
int scratch_device(int dev, ScratchDevice **out) {
    if (dev < 0 || dev >= kMaxDevices) return EP_ERR_ARG;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ScratchDevice &d = g_scratch_dev[dev];
    if (!d.ptr) {
        void *p = nullptr;
        if (int r = hip_fail(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress")) return r;
        if (!p) return EP_ERR_HIP;
        int cus = 0;
        if (int r = hip_fail(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev),
                             "hipDeviceGetAttribute"))
            return r;
        d.cu_count = cus;
        for (auto &plane : d.fused_per_cu)
            for (auto &row : plane) row[0] = row[1] = -1;
        const char *spin = std::getenv("EP_SPIN_LIMIT");
        d.spin_limit = spin ? (uint32_t)std::strtoul(spin, nullptr, 10) : kDefaultSpinLimit;
        const char *dbg = std::getenv("EP_DEBUG");
        d.debug = dbg && dbg[0] && dbg[0] != '0';
        d.ptr = p;
    }
    *out = &d;
    return EP_OK;
}

}  // namespace

extern "C" {

int ep_version(void) { return EP_ABI_VERSION; }

const char *ep_strerror(int code) {
    switch (code) {
        case EP_OK: return "ok";
        case EP_ERR_ARG: return "invalid argument";
        case EP_ERR_ALIGN: return "misaligned pointer (row arrays need 16-byte alignment)";
        case EP_ERR_HIP: return "HIP runtime error";
        case EP_ERR_NOMEM: return "out of device memory";
        case EP_ERR_SCRATCH: return "workload needs more workspace than the static scratch (4 MiB) of the no-allocation call";
        default: return "unknown error";
    }
}

int ep_query_sizes(const ep_config *cfg, ep_sizes *out) {
    if (int r = validate_config(cfg)) return r;
    if (!out) return EP_OK;
    const size_t T = cfg->num_tokens, k = cfg->num_topk, E = cfg->num_experts, R = cfg->num_ranks,
                 H = cfg->hidden, rows = R * (size_t)cfg->cap_rows;
    out->cnt_se = R * E * 4;
    out->cnt_sd = R * R * 4;
    out->recv_cnt = E * 4;
    out->expert_off = E * 4;
    out->rank_rows = R * 4;
    out->src_expert_off = R * E * 4;
    out->rank_in_expert = T * k * 4;
    out->is_token_in_rank = T * R;
    out->pos = T * k * 4;
    out->src_idx = rows * 4;
    out->x = T * H * 2;
    out->recv_x_bf16 = rows * H * 2;
    out->recv_x_fp8 = rows * H;
    out->recv_scales = rows * (H / 128) * 4;
    out->recv_w = rows * 4;
    out->combined_x = T * H * 2;
    out->rank_in_rank = T * k * 4;
    out->token_rows = R * 4;
    out->recv_topk_idx = rows * k * 4;
    out->recv_topk_w = rows * k * 4;
    out->workspace = workspace_layout(*cfg).total;
    return EP_OK;
}

int ep_create(const ep_config *cfg, ep_ctx **out) {
    if (!out) return EP_ERR_ARG;
    *out = nullptr;
    if (int r = validate_config(cfg)) return r;
    ep_ctx *ctx = new (std::nothrow) ep_ctx();
    if (!ctx) return EP_ERR_NOMEM;
    ctx->cfg = *cfg;
    ctx->num_tiles = num_tiles_of(*cfg);
    ctx->keys = cfg->num_experts + cfg->num_ranks;
    const WorkspaceLayout wl = workspace_layout(*cfg);
    ctx->ws_bytes = wl.total;
    const char *dbg = std::getenv("EP_DEBUG");
    ctx->debug = dbg && dbg[0] && dbg[0] != '0';
    const char *spin = std::getenv("EP_SPIN_LIMIT");
    ctx->spin_limit = spin ? (uint32_t)std::strtoul(spin, nullptr, 10) : kDefaultSpinLimit;
    if (hipGetDevice(&ctx->device) != hipSuccess ||
        hipDeviceGetAttribute(&ctx->cu_count, hipDeviceAttributeMultiprocessorCount, ctx->device) != hipSuccess) {
        delete ctx;
        return EP_ERR_HIP;
    }
    for (auto &plane : ctx->fused_per_cu)
        for (auto &row : plane) row[0] = row[1] = -1;
    ctx->cu_budget = 0;
    if (hipMalloc(&ctx->ws, ctx->ws_bytes) != hipSuccess) {
        delete ctx;
        return EP_ERR_NOMEM;
    }
    char *base = static_cast<char *>(ctx->ws);
    ctx->counters = reinterpret_cast<uint32_t *>(base);
    ctx->status = ctx->counters + ep::kStatus;
    ctx->tile_state = reinterpret_cast<uint64_t *>(base + wl.state);
    ctx->bp = reinterpret_cast<uint64_t *>(base + wl.bp);
    ctx->rank_ready = reinterpret_cast<uint32_t *>(base + wl.rank_ready);
    // all zero is the workspace's start: counters, and states and flags of
    // epoch 0, which no call uses
    int r = hip_fail(hipMemset(ctx->ws, 0, ctx->ws_bytes), "hipMemset");
    if (!r) r = hip_fail(hipDeviceSynchronize(), "hipDeviceSynchronize");
    if (r) {
        (void)hipFree(ctx->ws);
        delete ctx;
        return r;
    }
    if (ctx->debug)
        std::fprintf(stderr, "libep: ctx T=%d k=%d E=%d R=%d H=%d cap_rows=%lld tiles=%d workspace=%zu B\n",
                     cfg->num_tokens, cfg->num_topk, cfg->num_experts, cfg->num_ranks, cfg->hidden,
                     (long long)cfg->cap_rows, ctx->num_tiles, ctx->ws_bytes);
    *out = ctx;
    return EP_OK;
}

int ep_destroy(ep_ctx *ctx) {
    if (!ctx) return EP_OK;
    int r = hip_fail(hipDeviceSynchronize(), "hipDeviceSynchronize");
    if (hipFree(ctx->ws) != hipSuccess && !r) r = EP_ERR_HIP;
    delete ctx;
    return r;
}

int ep_get_dispatch_layout(ep_ctx *ctx, const int32_t *topk_idx, const ep_layout *L, ep_stream_t stream) {
    ep::LayoutArgs a;
    if (int r = fill_layout(ctx, topk_idx, L, a)) return r;
    if (ctx->debug)
        std::fprintf(stderr, "libep: layout T=%d k=%d E=%d R=%d tiles=%d\n", a.T, a.k, a.E, a.R, a.num_tiles);
    return hip_fail(ep::launch_layout(a, (hipStream_t)stream), "ep_get_dispatch_layout");
}

int ep_dispatch(ep_ctx *ctx, const uint16_t *x, const int32_t *topk_idx, const float *topk_weights,
                const ep_layout *L, int use_fp8, void *recv_x, float *recv_scales, float *recv_w,
                ep_handle *handle, ep_stream_t stream) {
    if (int r = check_forward_dispatch(ctx, topk_idx, topk_weights, L, use_fp8, recv_scales, recv_w, handle))
        return r;
    return dispatch_common(ctx, x, topk_idx, topk_weights, L, use_fp8 != 0, 1, recv_x, recv_scales, recv_w,
                           handle, stream, "ep_dispatch");
}

int ep_dispatch_dedup(ep_ctx *ctx, const uint16_t *x, const int32_t *topk_idx, const float *topk_weights,
                      const ep_layout *L, int use_fp8, void *recv_x, float *recv_scales, int32_t *recv_topk_idx,
                      float *recv_topk_w, ep_handle *handle, ep_stream_t stream) {
    if (int r = check_forward_dispatch(ctx, topk_idx, topk_weights, L, use_fp8, recv_scales, nullptr, handle))
        return r;
    const ep_config &c = ctx->cfg;
    if (c.num_tokens > 0 && !L->rank_in_rank) return EP_ERR_ARG;
    if (!recv_topk_idx && c.cap_rows > 0) return EP_ERR_ARG;
    if (recv_topk_w && !topk_weights) return EP_ERR_ARG;
    if (!aligned(recv_topk_idx, 4) || !aligned(recv_topk_w, 4)) return EP_ERR_ALIGN;
    return dispatch_common(ctx, x, topk_idx, topk_weights, L, use_fp8 != 0, 2, recv_x, recv_scales, nullptr,
                           handle, stream, "ep_dispatch_dedup", recv_topk_idx, recv_topk_w);
}

int ep_dispatch_low_latency(ep_ctx *ctx, const uint16_t *x, const int32_t *topk_idx, const float *topk_weights,
                            int use_fp8, void *recv_x, float *recv_scales, float *recv_w, int32_t *recv_count,
                            ep_handle *handle, ep_stream_t stream) {
    if (!ctx || !handle || !recv_count) return EP_ERR_ARG;
    if (int r = check_device(ctx)) return r;
    const ep_config &c = ctx->cfg;
    const int T = c.num_tokens, R = c.num_ranks;
    if (use_fp8 != 0 && use_fp8 != 1) return EP_ERR_ARG;
    if (use_fp8 && (c.hidden % 128 || !recv_scales)) return EP_ERR_ARG;
    if (!use_fp8 && recv_scales) return EP_ERR_ARG;
    // the low-latency receive layout: every expert holds T rows (R regions of T/R)
    if (c.cap_rows * R != (int64_t)c.num_experts * T || T / R > ep::kLayoutTile) return EP_ERR_ARG;
    if (T > 0 && (!topk_idx || !handle->pos || !handle->src_idx)) return EP_ERR_ARG;
    if (!aligned(recv_count, 4) || !aligned(topk_idx, 4) || !aligned(topk_weights, 4) || !aligned(recv_w, 4) ||
        !aligned(recv_scales, 4) || !aligned(handle->src_idx, 4))
        return EP_ERR_ALIGN;
    handle->num_tokens = T;
    handle->num_topk = c.num_topk;
    ep::DispatchArgs a;
    if (T == 0) {  // the region counts only
        std::memset(&a, 0, sizeof a);
        a.E = c.num_experts;
        a.k = c.num_topk;
        a.waves_per_token = 1;
        return hip_fail(ep::launch_ll_dispatch(a, false, R, recv_count, (hipStream_t)stream),
                        "ep_dispatch_low_latency");
    }
    Geometry g;
    if (int r = fill_dispatch(ctx, x, topk_idx, topk_weights, nullptr, 0, recv_x, recv_scales, recv_w, handle, a,
                              g))
        return r;
    return hip_fail(ep::launch_ll_dispatch(a, use_fp8 != 0, R, recv_count, (hipStream_t)stream),
                    "ep_dispatch_low_latency");
}

int ep_dispatch_dedup_with_layout(ep_ctx *ctx, const uint16_t *x, const int32_t *topk_idx,
                                  const float *topk_weights, const ep_layout *L, int use_fp8, void *recv_x,
                                  float *recv_scales, int32_t *recv_topk_idx, float *recv_topk_w, ep_handle *handle,
                                  ep_stream_t stream) {
    if (!ctx || !L || !L->token_rows) return EP_ERR_ARG;  // the deduplicated outputs are required
    ep::LayoutArgs la;
    if (int r = fill_layout(ctx, topk_idx, L, la)) return r;
    if (int r = check_forward_dispatch(ctx, topk_idx, topk_weights, L, use_fp8, recv_scales, nullptr, handle))
        return r;
    const ep_config &c = ctx->cfg;
    if (c.num_tokens == 0)  // nothing to pack: the layout alone (zero counts)
        return hip_fail(ep::launch_layout(la, (hipStream_t)stream), "ep_dispatch_dedup_with_layout");
    if (!recv_topk_idx && c.cap_rows > 0) return EP_ERR_ARG;
    if (recv_topk_w && !topk_weights) return EP_ERR_ARG;
    if (!aligned(recv_topk_idx, 4) || !aligned(recv_topk_w, 4)) return EP_ERR_ALIGN;
    ep::DispatchArgs da;
    Geometry g;
    if (int r = fill_dispatch(ctx, x, topk_idx, topk_weights, L, 2, recv_x, recv_scales, nullptr, handle, da, g))
        return r;
    da.recv_topk_idx = recv_topk_idx;
    da.recv_topk_w = topk_weights ? recv_topk_w : nullptr;
    return launch_fused(ctx, la, da, use_fp8 != 0, 2, g.num_waves, stream, "ep_dispatch_dedup_with_layout");
}

int ep_dispatch_with_layout(ep_ctx *ctx, const uint16_t *x, const int32_t *topk_idx, const float *topk_weights,
                            const ep_layout *L, int use_fp8, void *recv_x, float *recv_scales, float *recv_w,
                            ep_handle *handle, ep_stream_t stream) {
    return dispatch_with_layout(ctx, x, topk_idx, topk_weights, L, use_fp8, recv_x, recv_scales, recv_w, handle,
                                stream);
}

int ep_dispatch_with_layout_noalloc(const ep_config *cfg, const uint16_t *x, const int32_t *topk_idx,
                                    const float *topk_weights, const ep_layout *L, int use_fp8, void *recv_x,
                                    float *recv_scales, float *recv_w, ep_handle *handle, uint32_t *status,
                                    ep_stream_t stream) {
    if (int r = validate_config(cfg)) return r;
    if (!fits_scratch(*cfg)) return EP_ERR_SCRATCH;
    if (!aligned(status, 4)) return EP_ERR_ALIGN;
    int dev = -1;
    if (int r = hip_fail(hipGetDevice(&dev), "hipGetDevice")) return r;
    ScratchDevice *sd = nullptr;
    if (int r = scratch_device(dev, &sd)) return r;
    // a context on the stack over this device's static workspace
    ep_ctx ctx{};
    ctx.cfg = *cfg;
    ctx.device = dev;
    ctx.num_tiles = num_tiles_of(*cfg);
    ctx.keys = cfg->num_experts + cfg->num_ranks;
    ctx.ws = sd->ptr;
    ctx.ws_bytes = kScratchBytes;
    char *base = static_cast<char *>(sd->ptr);
    ctx.counters = reinterpret_cast<uint32_t *>(base);
    ctx.status = status ? status : ctx.counters + ep::kStatus;
    ctx.tile_state = reinterpret_cast<uint64_t *>(base + kScratchStates);
    ctx.bp = reinterpret_cast<uint64_t *>(base + kScratchBp);
    ctx.rank_ready = reinterpret_cast<uint32_t *>(base + kScratchRankReady);
    ctx.spin_limit = sd->spin_limit;
    ctx.debug = sd->debug;
    ctx.cu_count = sd->cu_count;
    ctx.cu_budget = 0;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        std::memcpy(ctx.fused_per_cu, sd->fused_per_cu, sizeof ctx.fused_per_cu);
    }
    const int r = dispatch_with_layout(&ctx, x, topk_idx, topk_weights, L, use_fp8, recv_x, recv_scales, recv_w,
                                       handle, stream);
    {  // keep what the call learned of the fused kernel's occupancy
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        std::memcpy(sd->fused_per_cu, ctx.fused_per_cu, sizeof ctx.fused_per_cu);
    }
    return r;
}

}  // extern "C"

namespace {

int dispatch_with_layout(ep_ctx *ctx, const uint16_t *x, const int32_t *topk_idx, const float *topk_weights,
                         const ep_layout *L, int use_fp8, void *recv_x, float *recv_scales, float *recv_w,
                         ep_handle *handle, ep_stream_t stream) {
    if (L && (L->rank_in_rank || L->token_rows)) return EP_ERR_ARG;  // per-expert rows only
    ep::LayoutArgs la;
    if (int r = fill_layout(ctx, topk_idx, L, la)) return r;
    if (int r = check_forward_dispatch(ctx, topk_idx, topk_weights, L, use_fp8, recv_scales, recv_w, handle))
        return r;
    const ep_config &c = ctx->cfg;
    if (c.num_tokens == 0)  // nothing to pack: the layout alone (zero counts)
        return hip_fail(ep::launch_layout(la, (hipStream_t)stream), "ep_dispatch_with_layout");
    ep::DispatchArgs da;
    Geometry g;
    if (int r = fill_dispatch(ctx, x, topk_idx, topk_weights, L, 1, recv_x, recv_scales, recv_w, handle, da, g))
        return r;
    if (ctx->debug)
        std::fprintf(stderr, "libep: layout+dispatch T=%d k=%d E=%d R=%d H=%d fp8=%d tiles=%d waves=%d\n", c.num_tokens,
                     c.num_topk, c.num_experts, c.num_ranks, c.hidden, use_fp8, ctx->num_tiles, g.num_waves);
    // One tile: every dispatch block builds the layout itself (no waits).
    // Otherwise the layout blocks raise flags the dispatch blocks wait on.
    const int keys = c.num_experts + c.num_ranks;
    if (ctx->num_tiles == 1 && ep::inblock_lds_bytes(keys, c.num_topk) <= ep::kMaxBlockLds)
        return hip_fail(ep::launch_dispatch_inblock(la, da, use_fp8 != 0, g.num_waves, (hipStream_t)stream),
                        "ep_dispatch_with_layout");
    return launch_fused(ctx, la, da, use_fp8 != 0, 1, g.num_waves, stream, "ep_dispatch_with_layout");
}

}  // namespace

extern "C" {

int ep_combine(ep_ctx *ctx, const uint16_t *expert_out, const ep_handle *handle, const float *weights,
               uint16_t *combined_x, ep_stream_t stream) {
    return combine_common(ctx, expert_out, handle, weights, combined_x, false, stream, "ep_combine");
}

int ep_combine_f32(ep_ctx *ctx, const uint16_t *expert_out, const ep_handle *handle, const float *weights,
                   float *combined_f32, ep_stream_t stream) {
    return combine_common(ctx, expert_out, handle, weights, combined_f32, true, stream, "ep_combine_f32");
}

int ep_prereduce(ep_ctx *ctx, const uint16_t *expert_out, const int32_t *recv_topk_idx, const float *recv_topk_w,
                 const int32_t *token_rows, uint16_t *reduced, ep_stream_t stream) {
    return prereduce_common(ctx, expert_out, recv_topk_idx, recv_topk_w, token_rows, reduced, false, stream,
                            "ep_prereduce");
}

int ep_prereduce_f32(ep_ctx *ctx, const uint16_t *expert_out, const int32_t *recv_topk_idx,
                     const float *recv_topk_w, const int32_t *token_rows, float *reduced_f32, ep_stream_t stream) {
    return prereduce_common(ctx, expert_out, recv_topk_idx, recv_topk_w, token_rows, reduced_f32, true, stream,
                            "ep_prereduce_f32");
}

int ep_combine_backward(ep_ctx *ctx, const uint16_t *grad_combined, const ep_handle *handle,
                        uint16_t *grad_rows, ep_stream_t stream) {
    if (!ctx) return EP_ERR_ARG;
    if (int r = check_device(ctx)) return r;
    if (int r = check_handle(ctx, handle)) return r;
    ep_handle h = *handle;
    return dispatch_common(ctx, grad_combined, nullptr, nullptr, nullptr, false, 0, grad_rows, nullptr,
                           nullptr, &h, stream, "ep_combine_backward");
}

int ep_dispatch_backward(ep_ctx *ctx, const uint16_t *grad_rows, const ep_handle *handle, const float *weights,
                         uint16_t *grad_x, ep_stream_t stream) {
    return combine_common(ctx, grad_rows, handle, weights, grad_x, false, stream, "ep_dispatch_backward");
}

int ep_get_status(ep_ctx *ctx, ep_stream_t stream, uint32_t *status) {
    if (!ctx || !status) return EP_ERR_ARG;
    if (int r = check_device(ctx)) return r;
    int r = hip_fail(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize");
    if (r) return r;
    r = hip_fail(hipMemcpy(status, ctx->counters + ep::kStatus, sizeof(uint32_t), hipMemcpyDeviceToHost),
                 "hipMemcpy");
    if (r) return r;
    const uint32_t zero = 0;
    return hip_fail(hipMemcpy(ctx->counters + ep::kStatus, &zero, sizeof zero, hipMemcpyHostToDevice), "hipMemcpy");
}

int ep_set_spin_limit(ep_ctx *ctx, uint32_t polls) {
    if (!ctx) return EP_ERR_ARG;
    ctx->spin_limit = polls ? polls : kDefaultSpinLimit;
    return EP_OK;
}

int ep_set_cu_budget(ep_ctx *ctx, int num_cus) {
    if (!ctx || num_cus < 0) return EP_ERR_ARG;
    ctx->cu_budget = num_cus;
    return EP_OK;
}

int ep_cu_mask(int cu_count, int num_cus, int exclude, uint32_t *mask, int words) {
    constexpr int kXcds = 8;
    if (!mask || cu_count <= 0 || cu_count % (8 * kXcds) || words < cu_count / 32) return EP_ERR_ARG;
    if (num_cus <= 0 || num_cus > cu_count || num_cus % kXcds || (exclude && num_cus == cu_count))
        return EP_ERR_ARG;
    // per XCD a, m units at offsets a*m .. a*m+m-1 (mod per): m per XCD when
    // bit i belongs to XCD i / per, and, since the 8m offsets run through
    // consecutive values and per is a multiple of 8, m per XCD when bit i
    // belongs to XCD i mod 8 as well
    const int per = cu_count / kXcds, m = num_cus / kXcds;
    for (int w = 0; w < words; ++w) mask[w] = 0;
    for (int a = 0; a < kXcds; ++a)
        for (int j = 0; j < m; ++j) {
            const int bit = a * per + (a * m + j) % per;
            mask[bit / 32] |= 1u << (bit % 32);
        }
    if (exclude)
        for (int w = 0; w < cu_count / 32; ++w) mask[w] = ~mask[w];
    return EP_OK;
}

int ep_stream_create_cus(int num_cus, int exclude, ep_stream_t *out) {
    if (!out) return EP_ERR_ARG;
    *out = nullptr;
    int dev = 0, cus = 0;
    if (int r = hip_fail(hipGetDevice(&dev), "hipGetDevice")) return r;
    if (int r = hip_fail(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev),
                         "hipDeviceGetAttribute"))
        return r;
    uint32_t mask[64];
    if (cus > 64 * 32) return EP_ERR_ARG;
    if (int r = ep_cu_mask(cus, num_cus, exclude, mask, cus / 32)) return r;
    hipStream_t s = nullptr;
    const hipError_t e = (!exclude && num_cus == cus) ? hipStreamCreate(&s)
                                                      : hipExtStreamCreateWithCUMask(&s, cus / 32, mask);
    if (int r = hip_fail(e, "hipExtStreamCreateWithCUMask")) return r;
    *out = s;
    return EP_OK;
}

int ep_stream_destroy(ep_stream_t stream) {
    if (!stream) return EP_OK;
    return hip_fail(hipStreamDestroy((hipStream_t)stream), "hipStreamDestroy");
}

int ep_cu_census(int blocks, int naps, uint32_t *ids, ep_stream_t stream) {
    if (blocks == 0) return EP_OK;
    if (blocks < 0 || blocks > (1 << 20) || naps < 0 || naps > 64 || !ids) return EP_ERR_ARG;
    if (!aligned(ids, 4)) return EP_ERR_ALIGN;
    return hip_fail(ep::launch_cu_census(blocks, naps, ids, (hipStream_t)stream), "ep_cu_census");
}

int ep_copy_bytes(const void *src, void *dst, size_t bytes, ep_stream_t stream) {
    if (bytes == 0) return EP_OK;
    if (!src || !dst || bytes % 16) return EP_ERR_ARG;
    if (!aligned(src, 16) || !aligned(dst, 16)) return EP_ERR_ALIGN;
    return hip_fail(ep::launch_copy(src, dst, bytes / 16, (hipStream_t)stream), "ep_copy_bytes");
}

}  // extern "C"
