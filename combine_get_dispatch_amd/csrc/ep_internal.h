// ep_internal.h -- kernel launch interface shared by ep_api.hip and ep_kernels.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ep {

// Layout scan geometry: one workgroup of 256 threads (4 waves) handles 256
// consecutive tokens, one token per lane; a single tile skips the cross-tile
// machinery. LDS per key: 4 wave masks (8 B), 4 wave prefixes, the tile's
// exclusive prefix and count, the expert scan (4 B each).
constexpr int kLayoutTile = 256;
constexpr int kCoResidentTiles = 256;  // grids up to this size number tiles by block index
constexpr int kLayoutReplicas = 8;     // blocks sharing the outputs of a single tile
inline size_t layout_lds_bytes(int keys) { return (size_t)keys * (4 * 8 + 4 * 4 + 3 * 4); }
// A fused launch on a single tile: every dispatch block builds the whole
// layout in its own LDS and keeps each slot's (expert, rank) beside it.
inline size_t inblock_lds_bytes(int keys, int k) { return layout_lds_bytes(keys) + (size_t)kLayoutTile * k * 4; }
constexpr size_t kMaxBlockLds = 64 * 1024;
constexpr int kMaxTopk = 32;
constexpr int kMaxRanks = 64;
constexpr int kMaxExperts = 1024;

// workspace counters (uint32 each). All zero is a valid start: the epoch
// counter holds the current epoch minus one. kStatus is the context's status
// word (kernels OR their status bits into the word `status` points at).
enum Counter { kTicket = 0, kDone = 1, kEpoch = 2, kStatus = 3, kTotalsReady = 4, kNumCounters = 16 };

struct LayoutArgs {
    const int32_t *topk;
    int T, k, E, R, epr, tpr, num_tiles;
    int epr_shift;   // log2(epr) when epr is a power of two, else -1
    int use_ticket;  // number tiles by start order (large grids) instead of block index
    int64_t cap_rows;
    int32_t *rank_in_expert;
    uint8_t *itr;
    int32_t *cnt_se, *cnt_sd, *recv_cnt, *expert_off, *rank_rows, *src_expert_off;
    uint64_t *tile_state;  // [num_tiles][E+R]
    uint64_t *bp;          // [R+1][E+R] prefixes at source-rank boundaries, tagged (epoch << 32 | prefix)
    uint32_t *rank_ready;  // [layout blocks] epoch once a block's ranks are written (fused launch)
    uint32_t *counters;
    uint32_t *status;  // sticky EP_ST_* bits
    uint32_t spin_limit;
    int32_t *rank_in_rank;  // [T][k] or NULL: the deduplicated exchange's rows (leader slots)
    int32_t *token_rows;    // [R] or NULL
};

struct DispatchArgs {
    const uint16_t *x;           // [T][H] bf16 (or grad_combined for combine_backward)
    const int32_t *topk;         // [T][k]        (forward only)
    const float *w;              // [T][k] or NULL (forward only)
    const int32_t *rank_in_expert;  // [T][k]     (forward only)
    const int32_t *expert_off;   // [E]           (forward only)
    const int32_t *rank_in_rank; // [T][k]        (deduplicated forward only)
    int32_t *recv_topk_idx;      // [R*cap][k]    (deduplicated forward only)
    float *recv_topk_w;          // [R*cap][k] or NULL (deduplicated forward only)
    int32_t *pos;                // [T][k] written (forward) or read (backward)
    int32_t *src_idx;            // [R*cap] (forward only)
    float *recv_w;               // [R*cap] or NULL (forward only)
    void *recv_x;                // [R*cap][H] e4m3 or bf16
    float *recv_scales;          // [R*cap][H/128] (FP8 only)
    int T, k, E, epr, epr_shift, H;
    int64_t cap_rows, num_rows;  // num_rows = R * cap_rows
    int waves_per_token, passes_per_wave, npass;
    uint32_t *counters;
    uint32_t *status;            // sticky EP_ST_* bits
};

struct CombineArgs {
    const uint16_t *rows;  // [R*cap][H] bf16 (pre-reduction: [R*cap][k][H], one row per (received row, slot))
    const int32_t *pos;    // [T][k] (pre-reduction: the rows' routing entries [R*cap][k], slot read if >= 0)
    const float *w;        // [T][k] or NULL
    void *out;             // [T][H] bf16 or fp32
    int T, k, H;           // (pre-reduction: T = R*cap received rows)
    int64_t num_rows;      // rows of `rows`; positions outside are skipped
    const int32_t *token_rows;  // pre-reduction: [R] used rows per rank
    int64_t cap_rows;           // pre-reduction: rows per rank
    int waves_per_token, passes_per_wave, npass;
    uint32_t *counters;
    uint32_t *status;      // sticky EP_ST_* bits
};

hipError_t launch_layout(const LayoutArgs &a, hipStream_t s);
// mode: 0 = backward (rows from handle positions), 1 = forward per expert,
// 2 = forward deduplicated per rank
hipError_t launch_dispatch(const DispatchArgs &a, bool fp8, int mode, int num_waves,
                           hipStream_t s);
hipError_t launch_dispatch_inblock(const LayoutArgs &la, const DispatchArgs &da, bool fp8, int num_waves,
                                   hipStream_t s);
// mode 1 (per expert) or 2 (deduplicated per rank; la.token_rows set);
// resident_blocks: blocks of the fused kernel the GPU holds at once (0: unknown)
hipError_t launch_layout_dispatch(const LayoutArgs &la, const DispatchArgs &da, bool fp8, int mode, int num_waves,
                                  int resident_blocks, hipStream_t s);
int layout_dispatch_blocks_per_cu(int k, bool fp8, int mode, size_t lds);
// prereduce: a.pos holds the received rows' routing entries and a.rows the
// per-(row, slot) expert outputs (see CombineArgs); its own kernel, which
// sizes its grid itself (num_waves is not used). cus: the device's compute
// units when the stream may use all of them, else 0 (no residency cap).
hipError_t launch_combine(const CombineArgs &a, bool out_f32, bool prereduce, int num_waves, int cus,
                          hipStream_t s);
hipError_t launch_copy(const void *src, void *dst, size_t n16, hipStream_t s);
hipError_t launch_cu_census(int blocks, int naps, uint32_t *ids, hipStream_t s);
// low-latency dispatch: a.T % R == 0, a.T / R <= kLayoutTile, rows e*T + s*(T/R) + r
size_t ll_lds_bytes(int E, int k, int tpr);
hipError_t launch_ll_dispatch(const DispatchArgs &a, bool fp8, int R, int32_t *recv_count, hipStream_t s);

}  // namespace ep
