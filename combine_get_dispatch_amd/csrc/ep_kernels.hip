// ep_kernels.hip -- gfx950 kernels of the MoE dispatch / combine hot path.
//
//   k_layout    dispatch layout: per-wave expert bitmasks in LDS (ds_or_b64)
//               and per-rank bitmasks from wave ballots, popcount ranks, and a
//               single-pass decoupled look-back scan (Merrill & Garland,
//               "Single-pass Parallel Prefix Scan with Decoupled Look-back",
//               2016) over per-tile expert/rank counts; each tile writes the
//               per-source outputs at the boundaries it owns and the last
//               tile the totals and offsets.
//   k_dispatch  token-major pack: each wave reads a token's row once with
//               128-bit non-temporal loads (branch-free buffer loads, so every
//               wait on the slot loads issued before them is exact; the
//               per-expert FP8 form issues them per pass) and writes it
//               to the token's k receive rows with 128-bit stores; in FP8
//               mode the per-128-channel amax is reduced across 8 lanes with
//               DPP and the row is packed with v_cvt_pk_fp8_f32 (OCP e4m3 on
//               gfx950).
//   k_combine   token-major gather-reduce: each wave loads the token's k rows
//               (all slots in flight, branch-free buffer loads, so each
//               slot's arithmetic waits only for its own rows) and
//               accumulates in fp32 with one fused
//               multiply-add per slot in slot order, then rounds to bf16;
//               a long launch runs at most 8 waves per CU (LDS reserved per
//               workgroup), which narrows the window of rows read at once.
//   k_prereduce expert-side pre-reduction of rank-deduplicated rows: several
//               received rows per wave, each row's valid slots summed in
//               slot order.
//   k_copy      plain 128-bit streaming copy (bandwidth calibration).
//   k_cu_census the compute unit each workgroup runs on (checks stream CU masks).
//   k_ll_dispatch low-latency dispatch: fixed per-(expert, source) regions, no
//               look-back, every block self-contained.
//
// The operations follow the DeepEP usage guide's dispatch / combine /
// backward interface (zhouruolin.cn DeepEP guide, section 5); the arithmetic
// each kernel implements is stated in include/ep.h.
#include "ep_internal.h"

namespace ep {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Buffer resources (gfx9 family): the fourth descriptor word of a raw,
// unswizzled buffer of 32-bit elements, and the cache-policy operand of a
// non-temporal load (bit 1).
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kLoadNonTemporal = 2;

constexpr uint32_t kStBad = 1u, kStDup = 2u, kStCap = 4u, kStTimeout = 8u, kStBadHandle = 16u;
constexpr int kWavesPerBlock = 4;
constexpr int kMaxPassPerWave = 8;  // dispatch: 1024 channels per pass

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (bias 0x7fff plus the kept lsb); NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// max with the value DPP control CTRL routes into this lane
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false)));
}

__device__ __forceinline__ int readlane_i(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// ---------------------------------------------------------------------------
// layout
// ---------------------------------------------------------------------------

// Look-back tile state: [63:34] epoch, [33:32] flag, [31:0] count. A word
// whose epoch differs from the current call's is "not yet published", so the
// states never need clearing between calls.
constexpr uint64_t kFlagAgg = 1, kFlagPrefix = 2;

__device__ __forceinline__ uint64_t pack_state(uint32_t epoch, uint64_t flag, uint32_t v) {
    return ((uint64_t)epoch << 34) | (flag << 32) | (uint64_t)v;
}

// Predecessor states read per round trip. Eight keep the layout kernels at
// 96 VGPRs and measured fastest on MI355X (same GPU, interleaved runs):
// standalone layout at 4096 tokens 13.7 us vs 14.4 (16 states) and 16.8
// (32); 16384 tokens as two launches 453.5 vs 458.4 us (32 states).
constexpr int kLookbackWindow = 8;
constexpr int kTileWaves = 4;
constexpr int kTileTokens = kTileWaves * 64;

// Exclusive prefix sum of one int per thread over a block of NW waves (wave
// scan with lane shuffles, then the wave totals). *total receives the sum.
template <int NW = kTileWaves>
__device__ __forceinline__ int block_exclusive_scan(int v, int *s_part, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) s_part[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < NW; ++w) {
            const int c = s_part[w];
            s_part[w] = run;
            run += c;
        }
        s_part[NW] = run;
    }
    __syncthreads();
    *total = s_part[NW];
    return s_part[wave] + x - v;
}

// One key's view of the tile, held in registers: the four wave masks.
struct KeyView {
    uint64_t m0, m1, m2, m3;
};

__device__ __forceinline__ KeyView key_view(const uint64_t *masks, int K, int key) {
    KeyView v;
    v.m0 = masks[key];
    v.m1 = masks[K + key];
    v.m2 = masks[2 * K + key];
    v.m3 = masks[3 * K + key];
    return v;
}

// Lanes [0, n) of a wave as a mask (n clamped to [0, 64]).
__device__ __forceinline__ uint64_t lanes_below(int n) {
    return n <= 0 ? 0ull : n >= 64 ? ~0ull : ((1ull << n) - 1);
}

// Tokens of this tile before tile-local position nb that hold the key
// (branch-free over the four waves, so the view stays in registers).
__device__ __forceinline__ int count_before(const KeyView &v, int nb, int ntile) {
    nb = min(nb, ntile);
    return __popcll(v.m0 & lanes_below(nb)) + __popcll(v.m1 & lanes_below(nb - 64)) +
           __popcll(v.m2 & lanes_below(nb - 128)) + __popcll(v.m3 & lanes_below(nb - 192));
}

// Four is_token_in_rank bytes (ranks d..d+3 of the mask, one byte each).
__device__ __forceinline__ uint32_t rank_bytes4(uint64_t rmask, int d) {
    const uint32_t x = (uint32_t)(rmask >> d) & 0xFu;
    return (x & 1u) | ((x & 2u) << 7) | ((x & 4u) << 14) | ((x & 8u) << 21);
}

// How a layout block runs: alone (its own grid), in a fused grid whose
// dispatch blocks wait on its readiness flags, or inside every dispatch block
// of a single-tile fused grid (the block keeps the whole layout in its LDS).
enum LayoutMode { kLayoutAlone = 0, kLayoutFlags = 1, kLayoutInBlock = 2 };

// Publishing to other blocks of the same grid. Everything a dispatch wave
// reads from the layout (ranks, expert offsets) is written with agent-scope
// stores, which are coherent across XCDs by themselves; a block releases them
// by having every thread wait until its stores are acknowledged (vmcnt also
// counts stores) before the barrier that precedes the flag store. This is the
// agent-scope release without the L2 write-back that plain stores would need
// (that write-back competes with the grid's row traffic for several us).
__device__ __forceinline__ void store_agent(int32_t *p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_own_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Expert e's rank: a shift when the experts per rank are a power of two.
__device__ __forceinline__ int rank_of(int e, int epr, int shift) { return shift >= 0 ? e >> shift : e / epr; }

// The layout's LDS, carved from the dynamic allocation (K = E + R keys).
struct LayoutLds {
    uint64_t *masks;  // [4 waves][K] token bitmasks per wave
    int32_t *wpre;    // [4][K] tokens in earlier waves
    int32_t *excl;    // [K] tokens in earlier tiles
    int32_t *agg;     // [K] tokens in this tile
    int32_t *scan;    // last tile: [E+1] prefix of expert rows (E + 1 <= K)
    int32_t *slots;   // in-block mode: [tile token][k] (expert << 16 | rank), -1 if not kept
};

__device__ __forceinline__ LayoutLds layout_lds(int K) {
    extern __shared__ uint64_t lds[];
    LayoutLds v;
    v.masks = lds;
    v.wpre = reinterpret_cast<int32_t *>(lds + kTileWaves * K);
    v.excl = v.wpre + kTileWaves * K;
    v.agg = v.excl + K;
    v.scan = v.agg + K;
    v.slots = v.scan + K;
    return v;
}

// The token's k slots (-1 past k or past the last token). The row index is
// clamped and every load issued, so that the wait for them is exact and the
// loads the caller issues next stay in flight.
template <int KMAX>
__device__ __forceinline__ void load_slots(const LayoutArgs &a, int t, int (&raw)[KMAX]) {
    const int tc = max(min(t, a.T - 1), 0);
    const int32_t *row = a.topk + (size_t)tc * a.k;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) raw[j] = row[min(j, a.k - 1)];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        if (t >= a.T || j >= a.k) raw[j] = -1;
}

// The call's epoch: the epoch counter plus one, so that a workspace filled
// with zeros is a valid start (no state or flag carries epoch 0). Epochs run
// through 1 .. 2^30 - 1 (30 bits of a look-back state word).
constexpr uint32_t kEpochPeriod = (1u << 30) - 1u;
__device__ __forceinline__ uint32_t load_epoch(const LayoutArgs &a) {
    return __hip_atomic_load(&a.counters[kEpoch], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
}

// One key's count in each wave of the tile and in the tile (LDS), published
// for the look-back of later tiles (tile 0's count is its inclusive prefix).
__device__ __forceinline__ void tile_counts(const uint64_t *masks, int32_t *wpre, int32_t *agg, const LayoutArgs &a,
                                            int K, int key, int tile, uint32_t epoch, bool single) {
    const int c0 = __popcll(masks[key]), c1 = __popcll(masks[K + key]), c2 = __popcll(masks[2 * K + key]),
              c3 = __popcll(masks[3 * K + key]);
    wpre[key] = 0;
    wpre[K + key] = c0;
    wpre[2 * K + key] = c0 + c1;
    wpre[3 * K + key] = c0 + c1 + c2;
    const int c = c0 + c1 + c2 + c3;
    agg[key] = c;
    if (!single)
        __hip_atomic_store(a.tile_state + (size_t)tile * K + key,
                           pack_state(epoch, tile == 0 ? kFlagPrefix : kFlagAgg, (uint32_t)c), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// What one tile's per-key look-back needs (registers and LDS of layout_block).
struct TileView {
    const LayoutArgs &a;
    const uint64_t *masks;
    const int32_t *agg;
    int32_t *excl;
    int K, tile;
    uint32_t epoch;
    bool single;
    int replica, nrep, t0, ntile, first_lo, first_hi;
};

// A boundary prefix as stored for other tiles: the call's epoch in the high
// word, so that a reader can tell this call's value from an older one.
__device__ __forceinline__ uint64_t tag_prefix(uint32_t epoch, int v) {
    return ((uint64_t)epoch << 32) | (uint32_t)v;
}

// Decoupled look-back of one key, a window of predecessors per round trip:
// add counts from the nearest predecessor back to the first inclusive
// prefix; a predecessor that has not published yet ends the window and is
// read again. Then this tile's share of the key's per-source outputs: one
// tile writes the per-source counts itself; several tiles store the key's
// prefix at each source-rank boundary they own (boundary s = token s*T/R)
// for the tiles that end those sources and for the last tile, which turns
// the expert keys' prefixes into src_expert_off. The tile's stores come
// after its look-back loads (stores and loads share one in-order completion
// counter).
__device__ __forceinline__ void lookback_key(const TileView &v, int key) {
    const LayoutArgs &a = v.a;
    const int K = v.K;
    int sum = 0;
    if (!v.single && v.tile > 0) {
        int hi = v.tile - 1;
        uint32_t spins = 0;
        while (hi >= 0) {
            uint64_t sv[kLookbackWindow];
#pragma unroll
            for (int i = 0; i < kLookbackWindow; ++i)
                sv[i] = (hi - i >= 0) ? __hip_atomic_load(a.tile_state + (size_t)(hi - i) * K + key,
                                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                      : 0ull;
            int consumed = 0;
            bool found = false, stall = false;
#pragma unroll
            for (int i = 0; i < kLookbackWindow; ++i) {
                if (found || stall || hi - i < 0) continue;
                const uint32_t fl = (uint32_t)(sv[i] >> 32) & 3u;
                if ((uint32_t)(sv[i] >> 34) != v.epoch || fl == 0) {
                    stall = true;
                    continue;
                }
                sum += (int32_t)(uint32_t)sv[i];
                ++consumed;
                if (fl == kFlagPrefix) found = true;
            }
            if (found) break;
            hi -= consumed;
            if (stall) {
                if (++spins > a.spin_limit) {
                    atomicOr(a.status, kStTimeout);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        __hip_atomic_store(a.tile_state + (size_t)v.tile * K + key,
                           pack_state(v.epoch, kFlagPrefix, (uint32_t)(sum + v.agg[key])), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    v.excl[key] = sum;
    const bool is_expert = key < a.E;
    const KeyView kv = key_view(v.masks, K, key);
    if (v.single) {
        // every boundary is here: per-source counts at once, the replicas
        // taking the source ranks in turn
        for (int s = v.replica; s < a.R; s += v.nrep) {
            const int lo = count_before(kv, s * a.tpr, v.ntile);
            const int hi = count_before(kv, (s + 1) * a.tpr, v.ntile);
            if (is_expert)
                a.cnt_se[(size_t)s * a.E + key] = hi - lo;
            else
                a.cnt_sd[(size_t)s * a.R + (key - a.E)] = hi - lo;
        }
    } else {
        for (int s = v.first_lo; s < v.first_hi; ++s)
            __hip_atomic_store(a.bp + (size_t)s * K + key,
                               tag_prefix(v.epoch, sum + count_before(kv, s * a.tpr - v.t0, v.ntile)),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Boundary prefixes read by other tiles of the same call: B words of bp per
// thread (entry u at offset at[u] when use[u]), all loads issued before the
// first wait. A word tagged with an older epoch is not yet written for this
// call and is read again (bounded, EP_ST_TIMEOUT); unused entries give 0.
template <int B>
__device__ __forceinline__ void load_prefixes(const LayoutArgs &a, const size_t (&at)[B], const bool (&use)[B],
                                              uint32_t epoch, int (&out)[B]) {
    uint64_t w[B];
#pragma unroll
    for (int u = 0; u < B; ++u)
        w[u] = use[u] ? __hip_atomic_load(a.bp + at[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                      : tag_prefix(epoch, 0);
#pragma unroll
    for (int u = 0; u < B; ++u) {
        uint32_t spins = 0;
        while ((uint32_t)(w[u] >> 32) != epoch) {
            if (++spins > a.spin_limit) {
                atomicOr(a.status, kStTimeout);
                w[u] = tag_prefix(epoch, 0);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            w[u] = __hip_atomic_load(a.bp + at[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        out[u] = (int32_t)(uint32_t)w[u];
    }
}

// The layout of tile `tile` (its 256 tokens are t0 + thread), given the
// thread's slots `raw` and the call's epoch. A single tile may run as `nrep`
// replicas that split the outputs (replica = this copy); several tiles chain
// through a decoupled look-back. In a fused launch the tile raises the flags
// the dispatch waves wait on.
template <int KMAX>
__device__ __forceinline__ void layout_block(const LayoutArgs &a, int tile, int replica, int nrep, int mode,
                                             const int (&raw)[KMAX], uint32_t epoch) {
    const int K = a.E + a.R;                   // keys: experts, then ranks
    const LayoutLds L = layout_lds(K);
    uint64_t *masks = L.masks;
    int32_t *wpre = L.wpre, *excl = L.excl, *agg = L.agg, *scan = L.scan;
    __shared__ int s_part[kTileWaves + 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool single = a.num_tiles == 1;
    const bool fused = mode == kLayoutFlags;
    const bool inblock = mode == kLayoutInBlock;  // (single tile only)

    const int t0 = tile * kTileTokens;
    const int t = t0 + tid;
    const int ntile = max(min(kTileTokens, a.T - t0), 0);  // tokens in this tile
    const bool last_tile = tile == a.num_tiles - 1;
    const uint64_t bit = 1ull << lane;
    // Source rank s holds tokens [s*T/R, (s+1)*T/R). This tile writes the
    // start offsets of the sources whose first token it holds, [first_lo,
    // first_hi), and the counts of those whose last token it holds,
    // [last_lo, last_hi); a source inside one tile needs nothing from others.
    int first_lo = 0, first_hi = 0, last_lo = 0, last_hi = 0;
    if (!single) {
        first_lo = min((t0 + a.tpr - 1) / a.tpr, a.R);
        first_hi = min((t0 + kTileTokens + a.tpr - 1) / a.tpr, a.R);
        last_lo = min(t0 / a.tpr, a.R);
        last_hi = min((t0 + kTileTokens) / a.tpr, a.R);
        if (last_tile) last_hi = a.R;
    }

    // each wave clears its own masks (LDS operations of a wave are ordered):
    // no barrier before the atomics
    for (int i = lane; i < K; i += 64) masks[wave * K + i] = 0;

    // 1. validate the token's slots; expert bits go into the wave's masks
    //    (LDS atomics); the token's ranks go into a register mask. One tile:
    //    the per-rank LDS masks are wave ballots of it (no atomics: every
    //    lane would hit the same few words). Several tiles: they are the ORs
    //    of their experts' masks, built in step 6, off the path to the ranks
    //    and the totals.
    int ev[KMAX];
    uint32_t st = 0;
    uint64_t rmask = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        ev[j] = -1;
        const int v = raw[j];
        if (v == -1) continue;
        if (v < -1 || v >= a.E) {
            st |= kStBad;
            continue;
        }
        bool dup = false;
#pragma unroll
        for (int jj = 0; jj < j; ++jj) dup |= (ev[jj] == v);
        if (dup) {
            st |= kStDup;
            continue;
        }
        ev[j] = v;
        atomicOr(reinterpret_cast<unsigned long long *>(&masks[wave * K + v]), (unsigned long long)bit);
        rmask |= 1ull << rank_of(v, a.epr, a.epr_shift);
    }
    if (single) {
        uint64_t mine = 0;
        for (int d = 0; d < a.R; ++d) {
            const uint64_t b = __ballot((rmask >> d) & 1);
            if (lane == d) mine = b;
        }
        if (lane < a.R) masks[wave * K + a.E + lane] = mine;
    }
    // tokens whose per-token outputs this block writes (all of them unless replicated)
    const int tok_chunk = (ntile + nrep - 1) / nrep;
    const bool my_token = t < a.T && tid >= replica * tok_chunk && tid < (replica + 1) * tok_chunk;
    if (st && replica == 0) atomicOr(a.status, st);
    __syncthreads();

    const TileView tv{a, masks, agg, excl, K, tile, epoch, single, replica, nrep, t0, ntile, first_lo, first_hi};
    const bool dedup = a.token_rows != nullptr;  // deduplicated rows asked for

    // The rank keys: masks (a token is on rank d if one of its kept slots'
    // experts is; one tile already has them from the ballots), counts and
    // look-back. Only the per-source counts and the deduplicated rows need
    // them.
    auto rank_keys = [&]() {
        if (!single) {
            for (int i = tid; i < kTileWaves * a.R; i += kTileTokens) {
                const int w = i / a.R, d = i - w * a.R;
                uint64_t m = 0;
                for (int e = d * a.epr; e < (d + 1) * a.epr; ++e) m |= masks[w * K + e];
                masks[w * K + a.E + d] = m;
            }
            __syncthreads();
            for (int key = a.E + tid; key < K; key += kTileTokens)
                tile_counts(masks, wpre, agg, a, K, key, tile, epoch, single);
        } else if (dedup) {
            for (int key = a.E + tid; key < K; key += kTileTokens)
                tile_counts(masks, wpre, agg, a, K, key, tile, epoch, single);
        }
        for (int key = a.E + tid; key < K; key += kTileTokens) lookback_key(tv, key);
    };

    // The deduplicated rows, when asked for (after the rank keys and a
    // barrier): the leader slot of each of the token's ranks (its first kept
    // slot there) gets the token's row in that rank, counted like the
    // per-expert ranks (earlier tiles, earlier waves, earlier lanes of the
    // rank's token mask); the last tile holds the totals. A fused grid then
    // raises the tile's flag: deduplicated rows need nothing else.
    auto dedup_rows = [&]() {
        if (my_token) {
            const uint64_t below = bit - 1;
            uint64_t led = 0;
            int rr[KMAX];
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                rr[j] = -1;
                if (ev[j] < 0) continue;
                const int d = rank_of(ev[j], a.epr, a.epr_shift);
                if ((led >> d) & 1) continue;
                led |= 1ull << d;
                const int key = a.E + d;
                rr[j] = excl[key] + wpre[wave * K + key] + __popcll(masks[wave * K + key] & below);
            }
            int32_t *out = a.rank_in_rank + (size_t)t * a.k;
            if (fused) {
#pragma unroll
                for (int j = 0; j < KMAX; ++j)
                    if (j < a.k) store_agent(out + j, rr[j]);
            } else if ((a.k & 3) == 0) {
#pragma unroll
                for (int j = 0; j < KMAX; j += 4)
                    if (j < a.k) *reinterpret_cast<int4 *>(out + j) = make_int4(rr[j], rr[j + 1], rr[j + 2], rr[j + 3]);
            } else {
#pragma unroll
                for (int j = 0; j < KMAX; ++j)
                    if (j < a.k) out[j] = rr[j];
            }
        }
        if (last_tile && replica == 0)
            for (int d = tid; d < a.R; d += kTileTokens) {
                const int rows = excl[a.E + d] + agg[a.E + d];
                a.token_rows[d] = rows;
                if ((int64_t)rows > a.cap_rows) atomicOr(a.status, kStCap);
            }
        if (fused) {
            wait_own_stores();
            __syncthreads();
            if (tid == 0)
                __hip_atomic_store(a.rank_ready + (single ? replica : tile), epoch, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    };

    // A fused grid of deduplicated rows does the rank keys first: its
    // dispatch waves wait for them alone.
    const bool rank_first = fused && dedup;
    if (rank_first) {
        rank_keys();
        __syncthreads();
        dedup_rows();
    }

    // 2. per expert key: tokens in earlier waves and the tile's count;
    //    published at once for the look-back (tile 0's count is already its
    //    inclusive prefix)
    for (int key = tid; key < a.E; key += kTileTokens) tile_counts(masks, wpre, agg, a, K, key, tile, epoch, single);

    // 3. decoupled look-back of the expert keys (the ranks and the totals
    //    wait on them); the rank keys, which only the per-source counts
    //    need, follow the ranks (step 6) so that no thread runs two chains
    //    before the totals.
    for (int key = tid; key < a.E; key += kTileTokens) lookback_key(tv, key);
    __syncthreads();

    // 4. the last tile holds every key's total (its look-back is done): rows
    //    per expert, expert offsets inside each rank (block scan), rows per
    //    rank. Replica 0 writes them, before its own ranks and per-source
    //    counts, which nothing waits on as long; the other copies of a single
    //    tile keep the scan for their share of src_expert_off (step 8), and
    //    in-block copies to place their own slots.
    if (last_tile && (replica == 0 || single)) {
        const int chunk = (a.E + kTileTokens - 1) / kTileTokens;
        const int lo = min(tid * chunk, a.E), hi = min(lo + chunk, a.E);
        int local = 0;
        for (int e = lo; e < hi; ++e) local += excl[e] + agg[e];
        int total;
        int run = block_exclusive_scan(local, s_part, &total);
        for (int e = lo; e < hi; ++e) {
            scan[e] = run;
            run += excl[e] + agg[e];
        }
        if (tid == 0) scan[a.E] = total;
        __syncthreads();
        if (replica == 0) {
            for (int e = tid; e < a.E; e += kTileTokens) {
                a.recv_cnt[e] = excl[e] + agg[e];
                store_agent(a.expert_off + e, scan[e] - scan[rank_of(e, a.epr, a.epr_shift) * a.epr]);
            }
            for (int d = tid; d < a.R; d += kTileTokens) {
                const int rows = scan[(d + 1) * a.epr] - scan[d * a.epr];
                a.rank_rows[d] = rows;
                if (!a.token_rows && (int64_t)rows > a.cap_rows) atomicOr(a.status, kStCap);
            }
            if (fused || !single) {
                // expert offsets are readable by the dispatch waves and the
                // src_expert_off block (several tiles) from here on
                wait_own_stores();
                __syncthreads();
                if (tid == 0)
                    __hip_atomic_store(&a.counters[kTotalsReady], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }

    // 5. stable rank of each kept slot: tokens before it in earlier tiles,
    //    earlier waves of this tile, and earlier lanes of its wave (in-block:
    //    every token's, kept in LDS for the block's dispatch waves)
    int r[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) r[j] = -1;
    if (my_token || (inblock && t < a.T)) {
        const uint64_t below = bit - 1;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const int e = ev[j];
            r[j] = e >= 0 ? excl[e] + wpre[wave * K + e] + __popcll(masks[wave * K + e] & below) : -1;
        }
        if (inblock) {
#pragma unroll
            for (int j = 0; j < KMAX; ++j)
                if (j < a.k) L.slots[tid * a.k + j] = ev[j] >= 0 ? (ev[j] << 16) | r[j] : -1;
        }
        if (my_token) {
            // is_token_in_rank row: R bytes, written with the widest aligned stores
            uint8_t *out = a.itr + (size_t)t * a.R;
            if ((a.R & 15) == 0) {
                for (int d = 0; d < a.R; d += 16) {
                    const u32x4 v4 = {rank_bytes4(rmask, d), rank_bytes4(rmask, d + 4), rank_bytes4(rmask, d + 8),
                                      rank_bytes4(rmask, d + 12)};
                    *reinterpret_cast<u32x4 *>(out + d) = v4;
                }
            } else if ((a.R & 7) == 0) {
                for (int d = 0; d < a.R; d += 8)
                    *reinterpret_cast<uint64_t *>(out + d) =
                        (uint64_t)rank_bytes4(rmask, d) | ((uint64_t)rank_bytes4(rmask, d + 4) << 32);
            } else if ((a.R & 3) == 0) {
                for (int d = 0; d < a.R; d += 4) *reinterpret_cast<uint32_t *>(out + d) = rank_bytes4(rmask, d);
            } else {
                for (int d = 0; d < a.R; ++d) out[d] = (uint8_t)((rmask >> d) & 1);
            }
            int32_t *rie = a.rank_in_expert + (size_t)t * a.k;
            if (fused) {
#pragma unroll
                for (int j = 0; j < KMAX; ++j)
                    if (j < a.k) store_agent(rie + j, r[j]);
            } else if ((a.k & 3) == 0) {
#pragma unroll
                for (int j = 0; j < KMAX; j += 4)
                    if (j < a.k) *reinterpret_cast<int4 *>(rie + j) = make_int4(r[j], r[j + 1], r[j + 2], r[j + 3]);
            } else {
#pragma unroll
                for (int j = 0; j < KMAX; ++j)
                    if (j < a.k) rie[j] = r[j];
            }
        }
    }

    // (a fused grid of deduplicated rows raised its flags with the rank keys)
    if (fused && !dedup) {
        // this block's ranks are readable by the dispatch waves from here on
        wait_own_stores();
        __syncthreads();
        if (tid == 0)
            __hip_atomic_store(a.rank_ready + (single ? replica : tile), epoch, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }

    // 6. the rank keys (unless done first, see above); their look-back also
    //    stores this tile's boundary prefixes of the rank keys. The workspace
    //    is re-armed by the last block of the grid to finish.
    if (!rank_first) rank_keys();
    __syncthreads();
    if (dedup && !rank_first) dedup_rows();

    // 7. per-source counts for the source ranks that end in this tile
    //    (source s = tokens [s*T/R, (s+1)*T/R)); a start boundary owned by an
    //    earlier tile is read back from the prefixes that tile stored
    if (!single && last_hi > last_lo) {
        const bool remote = last_lo * a.tpr < t0;  // only the first such source can start earlier
        int32_t *remote_lo = wpre;                 // [K] its start prefixes (wpre is free after step 5)
        if (remote) {
            __syncthreads();  // every wave is past step 5
            constexpr int kKeysPerThread = (kMaxExperts + kMaxRanks + kTileTokens - 1) / kTileTokens;
            size_t at[kKeysPerThread];
            bool use[kKeysPerThread];
            int pre[kKeysPerThread];
#pragma unroll
            for (int u = 0; u < kKeysPerThread; ++u) {
                at[u] = (size_t)last_lo * K + tid + u * kTileTokens;
                use[u] = tid + u * kTileTokens < K;
            }
            load_prefixes<kKeysPerThread>(a, at, use, epoch, pre);
#pragma unroll
            for (int u = 0; u < kKeysPerThread; ++u)
                if (use[u]) remote_lo[tid + u * kTileTokens] = pre[u];
        }
        for (int key = tid; key < K; key += kTileTokens) {
            const KeyView kv = key_view(masks, K, key);
            const int ex = excl[key];
            for (int s = last_lo; s < last_hi; ++s) {
                const int hi = ex + count_before(kv, (s + 1) * a.tpr - t0, ntile);
                const int lo = s * a.tpr >= t0 ? ex + count_before(kv, s * a.tpr - t0, ntile) : remote_lo[key];
                if (key < a.E)
                    a.cnt_se[(size_t)s * a.E + key] = hi - lo;
                else
                    a.cnt_sd[(size_t)s * a.R + (key - a.E)] = hi - lo;
            }
        }
    }

    // 8. src_expert_off[s][e]: where the rows source rank s sends to expert
    //    e start inside rank d(e)'s region, i.e. the expert's offset there
    //    (the scan of step 4) plus the rows of e from earlier sources. One
    //    tile has every boundary, its copies taking the sources in turn; of
    //    several tiles the last one writes it once its grid's other work is
    //    done (gather_src_expert_off).
    if (single) {
        for (int e = tid; e < a.E; e += kTileTokens) {
            const KeyView kv = key_view(masks, K, e);
            const int eo = scan[e] - scan[rank_of(e, a.epr, a.epr_shift) * a.epr];
            for (int s = replica; s < a.R; s += nrep)
                a.src_expert_off[(size_t)s * a.E + e] = eo + count_before(kv, s * a.tpr, ntile);
        }
    }
}

// src_expert_off of several tiles, by one extra block of the layout grid
// that follows the tiles in launch order (so everything it waits for is
// already running): once the last tile has published the expert offsets
// (the totals flag), the expert key's prefix at boundary s, which the
// boundary's owner stored in its look-back, plus the expert's offset in its
// rank. It overlaps the last tile's remaining work, and nothing on the
// dispatch path waits for it. Each thread takes experts tid, tid + 256, ...
// and loads sixteen boundaries' prefixes at a time before storing.
__device__ __forceinline__ void gather_src_expert_off(const LayoutArgs &a, uint32_t epoch) {
    const int tid = threadIdx.x, K = a.E + a.R;
    if (tid == 0) {
        uint32_t spins = 0;
        while (__hip_atomic_load(&a.counters[kTotalsReady], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
            if (++spins > a.spin_limit) {
                atomicOr(a.status, kStTimeout);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
    constexpr int kBatch = 16;
    for (int e = tid; e < a.E; e += kTileTokens) {
        const int eo = __hip_atomic_load(a.expert_off + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int s0 = 0; s0 < a.R; s0 += kBatch) {
            size_t at[kBatch];
            bool use[kBatch];
            int pre[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                at[u] = (size_t)(s0 + u) * K + e;
                use[u] = s0 + u < a.R && s0 + u > 0;  // boundary 0 is token 0: prefix 0
            }
            load_prefixes<kBatch>(a, at, use, epoch, pre);
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                if (s0 + u < a.R) a.src_expert_off[(size_t)(s0 + u) * a.E + e] = eo + pre[u];
        }
    }
}

// Which tile (and replica) a block of a layout grid computes; num_tiles: the
// src_expert_off block that follows several tiles; -1: none. Grids larger
// than the co-resident limit number tiles by start order (a ticket), so that
// every predecessor is already running.
__device__ __forceinline__ int layout_tile_of_block(const LayoutArgs &a, int b, int nblocks, int *replica, int *nrep) {
    __shared__ int s_tile;
    *replica = 0;
    *nrep = 1;
    if (a.num_tiles == 1) {
        *replica = b;
        *nrep = nblocks;
        return 0;
    }
    if (!a.use_ticket) return b;
    if (threadIdx.x == 0) s_tile = (int)atomicAdd(&a.counters[kTicket], 1u);
    __syncthreads();
    const int tile = s_tile;
    if (tile > a.num_tiles) {  // workspace not re-armed (an earlier call did not finish)
        if (threadIdx.x == 0) atomicOr(a.status, kStTimeout);
        return -1;
    }
    return tile;
}

// End of a layout or fused grid: the last block to finish re-arms the
// workspace (ticket, done counter, next epoch). Every block has read the
// epoch by then, so no block of this grid can tag its states with the next
// call's epoch, even when a bounded wait gave up.
__device__ __forceinline__ void rearm_workspace(const LayoutArgs &la) {
    __syncthreads();
    if (threadIdx.x == 0 && atomicAdd(&la.counters[kDone], 1u) == gridDim.x - 1) {
        const uint32_t c = __hip_atomic_load(&la.counters[kEpoch], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&la.counters[kTicket], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&la.counters[kDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&la.counters[kEpoch], (c + 1u) % kEpochPeriod, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int KMAX>
__global__ __launch_bounds__(kTileTokens) void k_layout(LayoutArgs a) {
    int replica, nrep;
    const int tile = layout_tile_of_block(a, (int)blockIdx.x, (int)gridDim.x, &replica, &nrep);
    if (tile >= 0 && tile < a.num_tiles) {  // uniform over the block
        int raw[KMAX];
        load_slots<KMAX>(a, tile * kTileTokens + (int)threadIdx.x, raw);
        const uint32_t epoch = load_epoch(a);  // (left in flight past the slots)
        layout_block<KMAX>(a, tile, replica, nrep, kLayoutAlone, raw, epoch);
    } else if (tile == a.num_tiles) {
        gather_src_expert_off(a, load_epoch(a));
    }
    rearm_workspace(a);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------

// What a dispatch wave of a fused launch waits for before reading the layout.
struct LayoutWait {
    const uint32_t *rank_ready;    // per layout block: epoch once its ranks are written
    const uint32_t *totals_ready;  // epoch once the expert offsets are written (NULL: not needed)
    uint32_t *status;
    uint32_t epoch, spin_limit;
    int tokens_per_block;          // tokens whose ranks one layout block writes
};

// One thread of the block polls the flags of the layout blocks that wrote
// the ranks of tokens [t_first, t_last] and the totals; the block waits at a
// barrier (few pollers: the flags are single words every block reads).
__device__ __forceinline__ void wait_for_layout(const LayoutWait &w, int t_first, int t_last) {
    if (threadIdx.x == 0) {
        const int lo = t_first / w.tokens_per_block, hi = t_last / w.tokens_per_block;
        uint32_t spins = 0;
        for (;;) {
            bool ready = !w.totals_ready ||
                         __hip_atomic_load(w.totals_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == w.epoch;
            for (int b = lo; b <= hi && ready; ++b)
                ready = __hip_atomic_load(w.rank_ready + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == w.epoch;
            if (ready) break;
            if (++spins > w.spin_limit) {
                atomicOr(w.status, kStTimeout);
                break;
            }
            __builtin_amdgcn_s_sleep(8);
        }
    }
    __syncthreads();
}

// How a dispatch wave finds its token's receive rows.
enum SlotMode { kRowsFromHandle = 0, kRowsPerExpert = 1, kRowsPerRank = 2 };

// Slot j's receive row lives in lane j (lanes >= k hold -1). Per expert: from
// the layout's ranks and expert offsets. Per rank (deduplicated): from the
// leader slots' ranks, and part 0 of the token also writes each kept row's
// routing entries. From the handle: the backward pass. In a fused launch the
// layout was written by other blocks of the same grid, so it is read with
// coherent (agent-scope) loads, after the wait for it.
//
// Loads and stores complete in issue order, so a wave that waits for one load
// also waits for every load issued before it. The lookup is therefore split
// in three: slot_inputs() loads what does not depend on a layout still being
// written (the routing entry, the weight and, outside a fused grid, the
// layout's rank) before the wave issues its row loads; slot_loads() issues
// the layout-dependent loads together (one round trip, not a chain of three);
// slot_finish() places the rows once they have arrived, with the FP8
// quantization in between.
struct SlotIn {
    int e;    // expert id (per expert, per rank) or the handle's position
    int r;    // rank within the expert / the rank (not fused), else -1
    float w;  // the slot's weight, when it is written to a receive buffer
};

struct SlotLd {
    int r;   // rank within the expert / the rank
    int eo;  // the expert's offset (per expert)
};

template <int MODE, bool FUSED>
__device__ __forceinline__ SlotIn slot_inputs(const DispatchArgs &a, int t, int lane) {
    SlotIn s{-1, -1, 0.0f};
    if (lane < a.k) {
        const size_t i = (size_t)t * a.k + lane;
        if (MODE == kRowsFromHandle) {
            s.e = a.pos[i];
        } else {
            s.e = a.topk[i];
            if (MODE == kRowsPerExpert ? a.recv_w != nullptr : a.recv_topk_w != nullptr) s.w = a.w[i];
            if (!FUSED) s.r = MODE == kRowsPerExpert ? a.rank_in_expert[i] : a.rank_in_rank[i];
        }
    }
    return s;
}

template <int MODE, bool FUSED>
__device__ __forceinline__ SlotLd slot_loads(const DispatchArgs &a, int t, int lane, const SlotIn &s) {
    SlotLd l{s.r, 0};
    if (MODE == kRowsFromHandle) return l;
    // every lane loads, lanes past k and invalid experts from a valid address
    // (their values are not used): with no branch around the loads, the wait
    // for them lands at their first use, after the quantization
    const size_t i = (size_t)t * a.k + min(lane, a.k - 1);
    const int32_t *ranks = MODE == kRowsPerExpert ? a.rank_in_expert : a.rank_in_rank;
    if (FUSED) l.r = __hip_atomic_load(ranks + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (MODE == kRowsPerExpert) {
        const int ec = (s.e >= 0 && s.e < a.E) ? s.e : 0;
        l.eo = FUSED ? __hip_atomic_load(a.expert_off + ec, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                     : a.expert_off[ec];
    }
    return l;
}

template <int MODE>
__device__ __forceinline__ int slot_finish(const DispatchArgs &a, int t, int lane, int part, const SlotIn &s,
                                           const SlotLd &l) {
    int p = -1;
    if (MODE == kRowsPerRank) {
        const size_t i = (size_t)t * a.k + lane;
        const int e = s.e, rr = l.r;
        int d = -1;
        // kept: a valid expert that no earlier slot of the token repeats (the
        // layout's rule), from the slots themselves
        int kept = e >= 0 && e < a.E;
        for (int jj = 0; jj < a.k; ++jj) {
            const int ej = readlane_i(e, jj);
            if (jj < lane && ej == e) kept = 0;
        }
        if (kept && rr >= 0) {
            d = rank_of(e, a.epr, a.epr_shift);
            if (rr < a.cap_rows) p = (int)((int64_t)d * a.cap_rows + rr);
        }
        if (part == 0) {
            if (lane < a.k) {
                a.pos[i] = p;
                if (p >= 0) a.src_idx[p] = t;
            }
            // the routing entries of the row this lane leads: slot jj's
            // expert index among rank d's experts, and its weight
            for (int jj = 0; jj < a.k; ++jj) {
                const int ej = readlane_i(e, jj), kj = readlane_i(kept, jj);
                const float wj = readlane_f(s.w, jj);
                if (p >= 0) {
                    const bool here = kj && rank_of(ej, a.epr, a.epr_shift) == d;
                    a.recv_topk_idx[(size_t)p * a.k + jj] = here ? ej - d * a.epr : -1;
                    if (a.recv_topk_w) a.recv_topk_w[(size_t)p * a.k + jj] = here ? wj : 0.0f;
                }
            }
        }
        return p;
    }
    if (lane < a.k) {
        const size_t i = (size_t)t * a.k + lane;
        if (MODE == kRowsPerExpert) {
            const int e = s.e, r = l.r;
            if (r >= 0 && e >= 0 && e < a.E) {
                const int64_t local = (int64_t)l.eo + r;
                if (local >= 0 && local < a.cap_rows)
                    p = (int)((int64_t)rank_of(e, a.epr, a.epr_shift) * a.cap_rows + local);
            }
            if (part == 0) {
                a.pos[i] = p;
                if (p >= 0) {
                    a.src_idx[p] = t;
                    if (a.recv_w) a.recv_w[p] = s.w;
                }
            }
        } else {
            p = s.e;
            if (p < -1 || p >= a.num_rows) {  // not a position this buffer holds
                atomicOr(a.status, kStBadHandle);
                p = -1;
            }
        }
    }
    return p;
}

// The bf16 source of this wave's passes, all loads issued at once (read
// once: non-temporal). FP8: 16 channels per lane per pass; BF16: two 8-channel
// vectors per lane, 512 channels apart. The loads go through a buffer
// resource spanning the token's row (none for an inactive wave): a load
// beyond it returns zeros without touching memory, so all 2*kMaxPassPerWave
// loads are issued with no branch around them. Loads complete in issue
// order, and with a fixed count between them the compiler's waits on the
// loads issued before the rows (the slots, the weight) no longer wait for
// the rows themselves. PPW (at least the wave's pass count) bounds the loads
// issued: a pass past it is not loaded at all, so a launch whose waves hold
// one pass each issues 2 loads, not 2 * kMaxPassPerWave.
template <bool FP8, int PPW = kMaxPassPerWave>
__device__ __forceinline__ void load_rows(const DispatchArgs &a, int t, int part, bool active,
                                          u32x4 (&v)[2 * kMaxPassPerWave]) {
    const int lane = threadIdx.x & 63;
    // t and active are the same in every lane of the wave
    const int tu = __builtin_amdgcn_readfirstlane(active ? t : 0);
    const int bytes = __builtin_amdgcn_readfirstlane(active ? a.H * 2 : 0);
    const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.x + (size_t)tu * a.H), 0, bytes, kBufferRsrcWord3);
    const int pass0 = part * a.passes_per_wave;
    const int np = min(a.passes_per_wave, a.npass - pass0);
#pragma unroll
    for (int i = 0; i < kMaxPassPerWave; ++i) {
        if (i >= PPW) {
            v[2 * i] = 0;
            v[2 * i + 1] = 0;
            continue;
        }
        const int ps = pass0 + i;
        // byte offsets of the lane's two vectors; past the row when the pass
        // is not this wave's
        int o0 = FP8 ? (ps * 1024 + lane * 16) * 2 : (ps * 1024 + lane * 8) * 2;
        int o1 = FP8 ? o0 + 16 : o0 + 1024;
        if (i >= np) o0 = o1 = bytes;
        v[2 * i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(row, o0, 0, kLoadNonTemporal));
        v[2 * i + 1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(row, o1, 0, kLoadNonTemporal));
    }
}

// The same loads with a wave-uniform branch per pass and a per-lane bounds
// test, so only the passes and vectors inside the row are issued, one
// branch apart, and the compiler's waits after them are for everything
// issued. In the forward per-expert FP8 dispatch run after a complete
// layout, which is bound by the HBM write rate of its scattered rows, this
// slower issue measured 60.2-61.2 us against 62.6-63.5 us for the
// branch-free loads at 4096 tokens x 7168 top-8 (same GPU, interleaved
// runs). The rank-deduplicated and gradient dispatches measured slower with
// it, and the fused and low-latency grids need the exact waits, so they keep
// the branch-free loader.
template <bool FP8>
__device__ __forceinline__ void load_rows_paced(const DispatchArgs &a, int t, int part,
                                                u32x4 (&v)[2 * kMaxPassPerWave]) {
    const int lane = threadIdx.x & 63;
    const int pass0 = part * a.passes_per_wave;
    const int np = min(a.passes_per_wave, a.npass - pass0);
    const int H = a.H;
    const uint16_t *xrow = a.x + (size_t)t * H;
#pragma unroll
    for (int i = 0; i < kMaxPassPerWave; ++i) {
        v[2 * i] = 0;
        v[2 * i + 1] = 0;
        if (i >= np) continue;
        const int ps = pass0 + i;
        if (FP8) {
            const int c = ps * 1024 + lane * 16;
            if (c < H) {
                const u32x4 *src = reinterpret_cast<const u32x4 *>(xrow + c);
                v[2 * i] = __builtin_nontemporal_load(src);
                v[2 * i + 1] = __builtin_nontemporal_load(src + 1);
            }
        } else {
            const int c0 = ps * 1024 + lane * 8;
            if (c0 < H) v[2 * i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xrow + c0));
            if (c0 + 512 < H)
                v[2 * i + 1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xrow + c0 + 512));
        }
    }
}

// FP8: quantize the wave's passes in place (pass i's 16 codes per lane into
// v[2i], its group scale into sc[i]). BF16 rows are copied as loaded.
template <bool FP8>
__device__ __forceinline__ void quantize_rows(const DispatchArgs &a, int part, u32x4 (&v)[2 * kMaxPassPerWave],
                                              float (&sc)[kMaxPassPerWave]) {
#pragma unroll
    for (int i = 0; i < kMaxPassPerWave; ++i) sc[i] = 0.0f;
    if (!FP8) return;
    const int np = min(a.passes_per_wave, a.npass - part * a.passes_per_wave);
#pragma unroll
    for (int i = 0; i < kMaxPassPerWave; ++i) {
        if (i >= np) continue;
        float f[16];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4 u = v[2 * i + h];
            f[8 * h + 0] = bf16_lo(u.x);
            f[8 * h + 1] = bf16_hi(u.x);
            f[8 * h + 2] = bf16_lo(u.y);
            f[8 * h + 3] = bf16_hi(u.y);
            f[8 * h + 4] = bf16_lo(u.z);
            f[8 * h + 5] = bf16_hi(u.z);
            f[8 * h + 6] = bf16_lo(u.w);
            f[8 * h + 7] = bf16_hi(u.w);
        }
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(f[e]));
        m = dpp_max<0xB1>(m);
        m = dpp_max<0x4E>(m);
        m = dpp_max<0x141>(m);
        const float am = fmaxf(m, 1e-4f);
        const float inv = 448.0f / am;   // IEEE division
        sc[i] = am / 448.0f;             // IEEE division
        uint32_t q[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float y0 = fminf(fmaxf(f[4 * e + 0] * inv, -448.0f), 448.0f);
            const float y1 = fminf(fmaxf(f[4 * e + 1] * inv, -448.0f), 448.0f);
            const float y2 = fminf(fmaxf(f[4 * e + 2] * inv, -448.0f), 448.0f);
            const float y3 = fminf(fmaxf(f[4 * e + 3] * inv, -448.0f), 448.0f);
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
            q[e] = (uint32_t)w;
        }
        v[2 * i] = u32x4{q[0], q[1], q[2], q[3]};
    }
}

// Write the wave's passes (quantized for FP8) into the receive rows of its
// token's kept slots (slot j's row in lane j of p). Rows are written with
// non-temporal stores. Ordinary stores are faster only while the rows stay
// in the 256 MB memory-side cache (MALL) from one call to the next, i.e.
// when the same receive buffer is rewritten with nothing in between; with
// independent buffers per step (as in a model, where every layer brings new
// data) the MI355X prefill step is 158.6 us with non-temporal row stores
// against 171.9 us with ordinary ones, and decode steps are no slower.
// Each destination row's passes are written back to back, which keeps a
// row's stores together in the memory queue (1024-token decode step 48.8 vs
// 50.5 us; prefill unchanged).
template <bool FP8>
__device__ __forceinline__ void write_rows(const DispatchArgs &a, int part, int p,
                                           const u32x4 (&v)[2 * kMaxPassPerWave],
                                           const float (&sc)[kMaxPassPerWave]) {
    const int lane = threadIdx.x & 63;
    const int pass0 = part * a.passes_per_wave;
    const int np = min(a.passes_per_wave, a.npass - pass0);
    const int H = a.H;
    if (FP8) {
        const int G = H >> 7;
        uint8_t *rx = static_cast<uint8_t *>(a.recv_x);
        // the wave's scales gathered so that lane L holds group pass0*8 + L
        // (pass L/8, group L%8; its value sits in the group's first lane):
        // one contiguous scale store per row instead of a 32-byte one per pass
        float scl = 0.0f;
#pragma unroll
        for (int i = 0; i < kMaxPassPerWave; ++i) {
            const float si = __shfl(sc[i], (lane & 7) << 3);
            if ((lane >> 3) == i) scl = si;
        }
        const int gl = pass0 * 8 + lane;
        const bool scale_lane = lane < np * 8 && gl < G;
        for (int j = 0; j < a.k; ++j) {
            const int pj = readlane_i(p, j);
            if (pj < 0) continue;
#pragma unroll
            for (int i = 0; i < kMaxPassPerWave; ++i) {
                if (i >= np) break;
                const int c = (pass0 + i) * 1024 + lane * 16;
                if (c < H) __builtin_nontemporal_store(v[2 * i], reinterpret_cast<u32x4 *>(rx + (size_t)pj * H + c));
            }
            if (scale_lane) a.recv_scales[(size_t)pj * G + gl] = scl;
        }
    } else {
        uint16_t *rx = static_cast<uint16_t *>(a.recv_x);
        for (int j = 0; j < a.k; ++j) {
            const int pj = readlane_i(p, j);
            if (pj < 0) continue;
#pragma unroll
            for (int i = 0; i < kMaxPassPerWave; ++i) {
                if (i >= np) break;
                const int c0 = (pass0 + i) * 1024 + lane * 8;
                u32x4 *dst = reinterpret_cast<u32x4 *>(rx + (size_t)pj * H + c0);
                if (c0 < H) __builtin_nontemporal_store(v[2 * i], dst);
                if (c0 + 512 < H) __builtin_nontemporal_store(v[2 * i + 1], dst + 64);
            }
        }
    }
}

template <bool FP8>
__device__ __forceinline__ void store_rows(const DispatchArgs &a, int part, int p, u32x4 (&v)[2 * kMaxPassPerWave]) {
    float sc[kMaxPassPerWave];
    quantize_rows<FP8>(a, part, v, sc);
    write_rows<FP8>(a, part, p, v, sc);
}

template <bool FP8, int MODE>
__global__ __launch_bounds__(kWavesPerBlock * 64) void k_dispatch(DispatchArgs a) {
    const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int t = gw / a.waves_per_token;
    const int part = gw - t * a.waves_per_token;
    if (t >= a.T) return;  // whole wave
    const int lane = threadIdx.x & 63;
    u32x4 v[2 * kMaxPassPerWave];
    float sc[kMaxPassPerWave];
    int p;
    if constexpr (FP8 && MODE == kRowsPerExpert) {
        // rows first, then the slots (see load_rows_paced)
        load_rows_paced<FP8>(a, t, part, v);
        const SlotIn s = slot_inputs<MODE, false>(a, t, lane);
        const SlotLd l = slot_loads<MODE, false>(a, t, lane, s);
        p = slot_finish<MODE>(a, t, lane, part, s, l);
        quantize_rows<FP8>(a, part, v, sc);
    } else {
        const SlotIn s = slot_inputs<MODE, false>(a, t, lane);  // issued before the rows
        load_rows<FP8>(a, t, part, true, v);
        __builtin_amdgcn_sched_barrier(0);  // every row load issued before the wait for the slots
        const SlotLd l = slot_loads<MODE, false>(a, t, lane, s);  // in flight during the quantization
        quantize_rows<FP8>(a, part, v, sc);
        p = slot_finish<MODE>(a, t, lane, part, s, l);
    }
    write_rows<FP8>(a, part, p, v, sc);
}

// Slot j's receive row (lane j) from the layout this block holds in LDS
// (in-block mode: single tile, so the token's index is its tile position).
__device__ __forceinline__ int slot_row_lds(const DispatchArgs &a, const LayoutLds &L, int t, int lane, int part,
                                            float wslot) {
    int p = -1;
    if (lane < a.k) {
        const int sv = L.slots[t * a.k + lane];
        if (sv >= 0) {
            const int e = sv >> 16, r = sv & 0xFFFF;
            const int d = rank_of(e, a.epr, a.epr_shift);
            const int64_t local = (int64_t)(L.scan[e] - L.scan[d * a.epr]) + r;
            if (local < a.cap_rows) p = (int)((int64_t)d * a.cap_rows + local);
        }
        if (part == 0) {
            const size_t i = (size_t)t * a.k + lane;
            a.pos[i] = p;
            if (p >= 0) {
                a.src_idx[p] = t;
                if (a.recv_w) a.recv_w[p] = wslot;
            }
        }
    }
    return p;
}

// Layout and forward dispatch of one tile (T <= 256) in one grid with no
// cross-block waits: every block loads its rows, builds the whole layout in
// LDS (writing its share of the layout outputs, like a replica), and places
// its rows from there.
template <int KMAX, bool FP8, int PPW>
__global__ __launch_bounds__(kTileTokens) void k_dispatch_inblock(LayoutArgs la, DispatchArgs da) {
    const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int t = gw / da.waves_per_token;
    const int part = gw - t * da.waves_per_token;
    const bool active = t < da.T;  // whole wave
    const int lane = threadIdx.x & 63;
    // loads before any store (stores share the in-order counter): the
    // slots the layout waits on first, the slot weight, then the rows
    int raw[KMAX];
    load_slots<KMAX>(la, (int)threadIdx.x, raw);
    const float wslot = (active && part == 0 && lane < da.k && da.recv_w) ? da.w[(size_t)t * da.k + lane] : 0.0f;
    u32x4 v[2 * kMaxPassPerWave];
    load_rows<FP8, PPW>(da, t, part, active, v);
    layout_block<KMAX>(la, 0, (int)blockIdx.x, (int)gridDim.x, kLayoutInBlock, raw, 0u);
    __syncthreads();  // the slots and the scan are in LDS
    if (!active) return;
    const int p = slot_row_lds(da, layout_lds(la.E + la.R), t, lane, part, wslot);
    store_rows<FP8>(da, part, p, v);
}

// Low-latency dispatch. Expert e's rows are R regions of tpr = T/R rows, one
// per source rank, so the row of a slot depends only on the tokens of its own
// source: slot (t, j) of source s with expert e lands in row
// e*R*tpr + s*tpr + (earlier tokens of s routed to e). Block b serves source
// s = b / bps: one thread per token of the source (tpr <= 256) validates its
// slots and ORs its bit into a per-wave 64-bit token mask of each of its
// experts in LDS; after one barrier every wave counts its slots' ranks with
// popcounts and writes its rows. No block waits on another and the context
// workspace is not used. The first block of each source writes the region
// counts recv_count[e][s].
template <int KMAX, bool FP8, int PPW>
__global__ __launch_bounds__(kTileTokens) void k_ll_dispatch(DispatchArgs da, int R, int tpr, int bps,
                                                            int32_t *__restrict__ recv_count) {
    extern __shared__ uint64_t ll_lds[];
    if (tpr == 0) {  // no tokens: empty regions
        for (int i = threadIdx.x; i < da.E * R; i += kTileTokens) recv_count[i] = 0;
        return;
    }
    const int nw = (tpr + 63) >> 6;                                   // waves holding the source's tokens
    uint64_t *masks = ll_lds;                                         // [nw][E] token bits per expert
    int *slots = reinterpret_cast<int *>(ll_lds + (size_t)nw * da.E);  // [tpr][k] kept expert or -1
    const int s = blockIdx.x / bps, bi = blockIdx.x - s * bps;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int item = bi * kWavesPerBlock + wave;
    const int tl = item / da.waves_per_token, part = item - tl * da.waves_per_token;
    const bool active = tl < tpr;  // whole wave
    const int t = s * tpr + (active ? tl : 0);
    // loads before any store: the source's slots (thread tid = its token tid),
    // the slot weight, then the rows
    int raw[KMAX];
    {
        const int32_t *row = da.topk + (size_t)(s * tpr + min(tid, tpr - 1)) * da.k;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) raw[j] = row[min(j, da.k - 1)];
    }
    const float wslot = (active && part == 0 && lane < da.k && da.recv_w) ? da.w[(size_t)t * da.k + lane] : 0.0f;
    u32x4 v[2 * kMaxPassPerWave];
    load_rows<FP8, PPW>(da, t, part, active, v);
    for (int i = tid; i < nw * da.E; i += kTileTokens) masks[i] = 0;
    uint32_t st = 0;
    int ev[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        ev[j] = -1;
        if (tid >= tpr || j >= da.k) continue;
        const int e = raw[j];
        if (e == -1) continue;
        if (e < 0 || e >= da.E) {
            st |= kStBad;
            continue;
        }
        bool dup = false;
#pragma unroll
        for (int jj = 0; jj < j; ++jj) dup |= raw[jj] == e;
        if (dup) {
            st |= kStDup;
            continue;
        }
        ev[j] = e;
    }
    __syncthreads();  // masks cleared
    const uint64_t bit = 1ull << lane;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
        if (ev[j] >= 0) atomicOr(reinterpret_cast<unsigned long long *>(masks + wave * da.E + ev[j]), bit);
    if (tid < tpr) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j < da.k) slots[tid * da.k + j] = ev[j];
    }
    if (st && bi == 0) atomicOr(da.status, st);
    __syncthreads();  // masks and slots complete
    if (bi == 0)
        for (int e = tid; e < da.E; e += kTileTokens) {
            int c = 0;
            for (int w = 0; w < nw; ++w) c += __popcll(masks[w * da.E + e]);
            recv_count[(size_t)e * R + s] = c;
        }
    if (!active) return;
    int p = -1;
    if (lane < da.k) {
        const int e = slots[tl * da.k + lane];
        if (e >= 0) {
            const int w0 = tl >> 6;
            int r = __popcll(masks[w0 * da.E + e] & ((1ull << (tl & 63)) - 1));
            for (int w = 0; w < w0; ++w) r += __popcll(masks[w * da.E + e]);
            p = (int)((int64_t)e * R * tpr + (int64_t)s * tpr + r);
        }
        if (part == 0) {
            const size_t i = (size_t)t * da.k + lane;
            da.pos[i] = p;
            if (p >= 0) {
                da.src_idx[p] = t;
                if (da.recv_w) da.recv_w[p] = wslot;
            }
        }
    }
    store_rows<FP8>(da, part, p, v);
}

// The dispatch side of a fused grid with flags: the block's NW waves load
// their routing entries and rows and (FP8) quantize the rows before the
// layout is known, wait for the layout blocks of their tokens and for the
// totals, load their slots' ranks and expert offsets together, then write
// the rows. `db` is the block's index among the dispatch blocks, which take
// the work items [0, items).
template <bool FP8, int NW, int MODE>
__device__ __forceinline__ void fused_dispatch_block(const DispatchArgs &da, const LayoutWait &lw, int db, int items) {
    const int gw = db * NW + (int)(threadIdx.x >> 6);
    const int t = gw / da.waves_per_token;
    const int part = gw - t * da.waves_per_token;
    const bool active = gw < items;  // whole wave
    const int lane = threadIdx.x & 63;
    SlotIn s{-1, -1, 0.0f};
    if (active) s = slot_inputs<MODE, true>(da, t, lane);
    u32x4 v[2 * kMaxPassPerWave];
    load_rows<FP8>(da, t, part, active, v);  // loaded and quantized before the layout is known
    float sc[kMaxPassPerWave];
    quantize_rows<FP8>(da, part, v, sc);
    // every wave of the block reaches the barrier inside
    const int gw0 = db * NW;
    const int t_first = min(gw0 / da.waves_per_token, da.T - 1);
    const int t_last = min((min(gw0 + NW, items) - 1) / da.waves_per_token, da.T - 1);
    wait_for_layout(lw, t_first, max(t_last, t_first));
    if (active) {
        const SlotLd l = slot_loads<MODE, true>(da, t, lane, s);
        const int p = slot_finish<MODE>(da, t, lane, part, s, l);
        write_rows<FP8>(da, part, p, v, sc);
    }
}

// One wave waits for the layout block that wrote token t's ranks and for
// the totals (a layout wave taking a dispatch item after its layout work).
__device__ __forceinline__ void wave_wait_for_layout(const LayoutWait &w, int t) {
    const uint32_t *flag = w.rank_ready + t / w.tokens_per_block;
    uint32_t spins = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != w.epoch ||
           (w.totals_ready &&
            __hip_atomic_load(w.totals_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != w.epoch)) {
        if (++spins > w.spin_limit) {
            atomicOr(w.status, kStTimeout);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

__device__ __forceinline__ LayoutWait make_wait(const LayoutArgs &la, uint32_t epoch, int tokens_per_block,
                                                bool totals) {
    LayoutWait lw;
    lw.rank_ready = la.rank_ready;
    lw.totals_ready = totals ? la.counters + kTotalsReady : nullptr;
    lw.status = la.status;
    lw.epoch = epoch;
    lw.spin_limit = la.spin_limit;
    lw.tokens_per_block = max(tokens_per_block, 1);
    return lw;
}

// Layout and forward dispatch in one grid: blocks [0, lgrid) compute the
// layout (the tiles, or the replicas of one tile), the rest are dispatch
// waves that load and quantize their rows first and wait for the layout only
// to place them. Layout blocks have the lowest indices, so they are running
// before any dispatch block waits. When the grid would not fit on the GPU at
// once, the last `extra` work items (at most four per layout block) go to the
// layout blocks' own waves once their layout work is done, so that no
// dispatch block has to wait for a free slot (it would then run its chain of
// dependent loads behind everyone's row traffic). Not with a ticket: then
// the layout blocks themselves need the slots their predecessors free.
// Top-8 grids are held to 5 waves per SIMD (at most 102 VGPRs; 96 with the
// 8-state look-back, no spills), so the whole prefill grid is resident at
// once: 62.1 vs 63.3 us at 4096 tokens x 7168 top-8 with 4 waves per SIMD
// (same GPU, interleaved runs). Wider top-k keeps its registers.
template <int KMAX, bool FP8, int MODE>
__global__ __launch_bounds__(kTileTokens) __attribute__((amdgpu_waves_per_eu(KMAX <= 8 ? 5 : 1, 8))) void
k_layout_dispatch(LayoutArgs la, DispatchArgs da, int lgrid, int extra) {
    // per expert: ranks and expert offsets (the totals); per rank: leader rows only
    constexpr bool kTotals = MODE == kRowsPerExpert;
    const int b = (int)blockIdx.x;
    const int items = da.T * da.waves_per_token;
    const int tpb = la.num_tiles > 1 ? kTileTokens : (la.T + lgrid - 1) / lgrid;
    if (b < lgrid) {
        int replica, nrep;
        const int tile = layout_tile_of_block(la, b, lgrid, &replica, &nrep);
        uint32_t epoch = 0;
        if (tile >= 0) {
            int raw[KMAX];
            load_slots<KMAX>(la, tile * kTileTokens + (int)threadIdx.x, raw);
            epoch = load_epoch(la);
            layout_block<KMAX>(la, tile, replica, nrep, kLayoutFlags, raw, epoch);
        } else {
            epoch = load_epoch(la);
        }
        const int lw = b * kWavesPerBlock + (int)(threadIdx.x >> 6);
        const int gw = items - extra + lw;
        const int t = gw / da.waves_per_token;
        if (lw < extra) {  // whole wave
            const int part = gw - t * da.waves_per_token;
            const int lane = threadIdx.x & 63;
            const SlotIn s = slot_inputs<MODE, true>(da, t, lane);
            u32x4 v[2 * kMaxPassPerWave];
            load_rows<FP8>(da, t, part, true, v);
            float sc[kMaxPassPerWave];
            quantize_rows<FP8>(da, part, v, sc);
            wave_wait_for_layout(make_wait(la, epoch, tpb, kTotals), t);
            const SlotLd l = slot_loads<MODE, true>(da, t, lane, s);
            const int p = slot_finish<MODE>(da, t, lane, part, s, l);
            write_rows<FP8>(da, part, p, v, sc);
        }
    } else if (la.num_tiles > 1 && b == (int)gridDim.x - 1) {
        // the src_expert_off block, last in the grid (it starts once a slot
        // frees; everything it waits for runs before it)
        gather_src_expert_off(la, load_epoch(la));
    } else {
        const uint32_t epoch = load_epoch(la);
        fused_dispatch_block<FP8, kWavesPerBlock, MODE>(da, make_wait(la, epoch, tpb, kTotals), b - lgrid,
                                                        items - extra);
    }
    rearm_workspace(la);
}

// ---------------------------------------------------------------------------
// combine
// ---------------------------------------------------------------------------

constexpr int kSlotChunk = 8;
constexpr size_t kCombineCapLds = 40 * 1024;  // 4 two-wave workgroups in a CU's 160 KB of LDS
constexpr int kCombineCapMinWavesPerCu = 64;

template <bool OUT_F32, int WPB>
__global__ __launch_bounds__(WPB * 64) void k_combine(CombineArgs a) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * WPB + (threadIdx.x >> 6);
    const int t = gw / a.waves_per_token;
    const int part = gw - t * a.waves_per_token;
    if (t >= a.T) return;

    int p = -1;
    float wt = 1.0f;
    if (lane < a.k) {
        p = a.pos[(size_t)t * a.k + lane];
        if (p < -1 || p >= a.num_rows) {  // not a position this buffer holds
            atomicOr(a.status, kStBadHandle);
            p = -1;
        }
        if (a.w) wt = a.w[(size_t)t * a.k + lane];
    }
    const int H = a.H;
    const int pass0 = part * a.passes_per_wave;
    const int pass1 = min(pass0 + a.passes_per_wave, a.npass);

    for (int ps = pass0; ps < pass1; ++ps) {
        const int c0 = ps * 1024 + lane * 8;  // channels c0..c0+7 and c0+512..c0+519
        const bool a0 = c0 < H, a1 = c0 + 512 < H;
        float acc0[8], acc1[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc0[e] = 0.0f;
            acc1[e] = 0.0f;
        }
        for (int jb = 0; jb < a.k; jb += kSlotChunk) {
            u32x4 r0[kSlotChunk], r1[kSlotChunk];
            int pj[kSlotChunk];
            float wj[kSlotChunk];
#pragma unroll
            for (int jj = 0; jj < kSlotChunk; ++jj) {
                const int j = jb + jj;
                pj[jj] = j < a.k ? readlane_i(p, j) : -1;
                wj[jj] = readlane_f(wt, j & 63);
                // the slot's row as a buffer resource (none for an empty
                // slot): a vector past it reads zeros without touching
                // memory, so every load is issued with no branch around it
                // and each slot's multiply-adds wait only for that slot
                const int pr = max(pj[jj], 0);
                const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<uint16_t *>(a.rows + (size_t)pr * H), 0, pj[jj] >= 0 ? H * 2 : 0, kBufferRsrcWord3);
                r0[jj] = __builtin_bit_cast(u32x4,
                                            __builtin_amdgcn_raw_buffer_load_b128(row, c0 * 2, 0, kLoadNonTemporal));
                r1[jj] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(row, c0 * 2 + 1024, 0, kLoadNonTemporal));
            }
#pragma unroll
            for (int jj = 0; jj < kSlotChunk; ++jj) {
                if (pj[jj] < 0) continue;
                const float w = wj[jj];
                const u32x4 u = r0[jj], z = r1[jj];
                acc0[0] = __builtin_fmaf(w, bf16_lo(u.x), acc0[0]);
                acc0[1] = __builtin_fmaf(w, bf16_hi(u.x), acc0[1]);
                acc0[2] = __builtin_fmaf(w, bf16_lo(u.y), acc0[2]);
                acc0[3] = __builtin_fmaf(w, bf16_hi(u.y), acc0[3]);
                acc0[4] = __builtin_fmaf(w, bf16_lo(u.z), acc0[4]);
                acc0[5] = __builtin_fmaf(w, bf16_hi(u.z), acc0[5]);
                acc0[6] = __builtin_fmaf(w, bf16_lo(u.w), acc0[6]);
                acc0[7] = __builtin_fmaf(w, bf16_hi(u.w), acc0[7]);
                acc1[0] = __builtin_fmaf(w, bf16_lo(z.x), acc1[0]);
                acc1[1] = __builtin_fmaf(w, bf16_hi(z.x), acc1[1]);
                acc1[2] = __builtin_fmaf(w, bf16_lo(z.y), acc1[2]);
                acc1[3] = __builtin_fmaf(w, bf16_hi(z.y), acc1[3]);
                acc1[4] = __builtin_fmaf(w, bf16_lo(z.z), acc1[4]);
                acc1[5] = __builtin_fmaf(w, bf16_hi(z.z), acc1[5]);
                acc1[6] = __builtin_fmaf(w, bf16_lo(z.w), acc1[6]);
                acc1[7] = __builtin_fmaf(w, bf16_hi(z.w), acc1[7]);
            }
        }
        if (OUT_F32) {
            float *out = static_cast<float *>(a.out) + (size_t)t * H + c0;
            if (a0) {
                u32x4 o0 = {__float_as_uint(acc0[0]), __float_as_uint(acc0[1]), __float_as_uint(acc0[2]),
                            __float_as_uint(acc0[3])};
                u32x4 o1 = {__float_as_uint(acc0[4]), __float_as_uint(acc0[5]), __float_as_uint(acc0[6]),
                            __float_as_uint(acc0[7])};
                reinterpret_cast<u32x4 *>(out)[0] = o0;
                reinterpret_cast<u32x4 *>(out)[1] = o1;
            }
            if (a1) {
                u32x4 o0 = {__float_as_uint(acc1[0]), __float_as_uint(acc1[1]), __float_as_uint(acc1[2]),
                            __float_as_uint(acc1[3])};
                u32x4 o1 = {__float_as_uint(acc1[4]), __float_as_uint(acc1[5]), __float_as_uint(acc1[6]),
                            __float_as_uint(acc1[7])};
                reinterpret_cast<u32x4 *>(out + 512)[0] = o0;
                reinterpret_cast<u32x4 *>(out + 512)[1] = o1;
            }
        } else {
            uint16_t *out = static_cast<uint16_t *>(a.out) + (size_t)t * H + c0;
            if (a0) {
                const u32x4 o = {bf16_rne(acc0[0]) | (bf16_rne(acc0[1]) << 16),
                                 bf16_rne(acc0[2]) | (bf16_rne(acc0[3]) << 16),
                                 bf16_rne(acc0[4]) | (bf16_rne(acc0[5]) << 16),
                                 bf16_rne(acc0[6]) | (bf16_rne(acc0[7]) << 16)};
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(out));
            }
            if (a1) {
                const u32x4 o = {bf16_rne(acc1[0]) | (bf16_rne(acc1[1]) << 16),
                                 bf16_rne(acc1[2]) | (bf16_rne(acc1[3]) << 16),
                                 bf16_rne(acc1[4]) | (bf16_rne(acc1[5]) << 16),
                                 bf16_rne(acc1[6]) | (bf16_rne(acc1[7]) << 16)};
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(out + 512));
            }
        }
    }
}

// Expert-side pre-reduction of rank-deduplicated rows, M consecutive
// received rows per wave (one 1024-channel pass of each): lanes l < M*k load
// the routing entry of row r0 + l/k, slot l%k, and whether that row is used
// (row p of rank d = p / cap_rows is used below token_rows[d]); a ballot gives
// the valid (row, slot) pairs in row-major slot order, whose expert outputs
// (entry p*k + j of the per-(row, slot) outputs) are loaded C at a time
// through buffer resources and summed per row with one fused multiply-add per
// slot in slot order, then rounded to bf16 (or kept fp32) and written for the
// used rows. One routing round trip serves M rows, so a wave keeps M times
// the bytes of a one-row wave in flight.
template <bool OUT_F32, int M, int C>
__global__ __launch_bounds__(kWavesPerBlock * 64) void k_prereduce(CombineArgs a) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int grp = gw / a.npass, ps = gw - grp * a.npass;
    const int r0 = grp * M;
    if (r0 >= a.T) return;  // whole wave
    const int k = a.k, H = a.H;
    const int lr = lane / k, ls = lane - lr * k;
    const int row = r0 + lr;
    const bool mine = lr < M && row < a.T;
    // the row's used flag and its routing entry, loaded together
    const int rc = mine ? row : r0;
    const int d = (int)(rc / a.cap_rows);
    const int tr = a.token_rows[d];
    const int e = a.pos[(size_t)rc * k + (mine ? ls : 0)];
    const float wt = (a.w && mine) ? a.w[(size_t)rc * k + ls] : 1.0f;
    const bool used = mine && (int64_t)rc - (int64_t)d * a.cap_rows < (int64_t)tr;
    const uint64_t valid = __ballot(used && e >= 0);
    const uint64_t used_lanes = __ballot(used && ls == 0);
    const int c0 = ps * 1024 + lane * 8;  // channels c0..c0+7 and c0+512..c0+519
    float acc[M][16];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][i] = 0.0f;
    uint64_t rem = valid;
    while (rem) {  // wave-uniform
        int pl[C];
        u32x4 v0[C], v1[C];
#pragma unroll
        for (int q = 0; q < C; ++q) {
            pl[q] = rem ? __builtin_ctzll(rem) : -1;
            rem &= rem - 1;  // (0 stays 0)
            const int ll = max(pl[q], 0);
            const int rr = r0 + ll / k, ss = ll - (ll / k) * k;
            const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t *>(a.rows + ((size_t)rr * k + ss) * H), 0, pl[q] >= 0 ? H * 2 : 0,
                kBufferRsrcWord3);
            v0[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src, c0 * 2, 0, kLoadNonTemporal));
            v1[q] = __builtin_bit_cast(u32x4,
                                       __builtin_amdgcn_raw_buffer_load_b128(src, c0 * 2 + 1024, 0, kLoadNonTemporal));
        }
#pragma unroll
        for (int q = 0; q < C; ++q) {
            if (pl[q] < 0) continue;  // uniform
            const float w = readlane_f(wt, pl[q]);
            const int m = pl[q] / k;
            const u32x4 u = v0[q], z = v1[q];
            const float f[16] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                                 bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w),
                                 bf16_lo(z.x), bf16_hi(z.x), bf16_lo(z.y), bf16_hi(z.y),
                                 bf16_lo(z.z), bf16_hi(z.z), bf16_lo(z.w), bf16_hi(z.w)};
#pragma unroll
            for (int mm = 0; mm < M; ++mm) {
                if (mm != m) continue;  // uniform
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mm][i] = __builtin_fmaf(w, f[i], acc[mm][i]);
            }
        }
    }
    const bool a0 = c0 < H, a1 = c0 + 512 < H;
#pragma unroll
    for (int mm = 0; mm < M; ++mm) {
        if (!((used_lanes >> (mm * k)) & 1)) continue;  // row not used (uniform)
        const size_t base = (size_t)(r0 + mm) * H + c0;
        if (OUT_F32) {
            float *out = static_cast<float *>(a.out) + base;
            if (a0) {
                reinterpret_cast<u32x4 *>(out)[0] = u32x4{__float_as_uint(acc[mm][0]), __float_as_uint(acc[mm][1]),
                                                          __float_as_uint(acc[mm][2]), __float_as_uint(acc[mm][3])};
                reinterpret_cast<u32x4 *>(out)[1] = u32x4{__float_as_uint(acc[mm][4]), __float_as_uint(acc[mm][5]),
                                                          __float_as_uint(acc[mm][6]), __float_as_uint(acc[mm][7])};
            }
            if (a1) {
                reinterpret_cast<u32x4 *>(out + 512)[0] =
                    u32x4{__float_as_uint(acc[mm][8]), __float_as_uint(acc[mm][9]), __float_as_uint(acc[mm][10]),
                          __float_as_uint(acc[mm][11])};
                reinterpret_cast<u32x4 *>(out + 512)[1] =
                    u32x4{__float_as_uint(acc[mm][12]), __float_as_uint(acc[mm][13]), __float_as_uint(acc[mm][14]),
                          __float_as_uint(acc[mm][15])};
            }
        } else {
            uint16_t *out = static_cast<uint16_t *>(a.out) + base;
            if (a0)
                __builtin_nontemporal_store(
                    u32x4{bf16_rne(acc[mm][0]) | (bf16_rne(acc[mm][1]) << 16),
                          bf16_rne(acc[mm][2]) | (bf16_rne(acc[mm][3]) << 16),
                          bf16_rne(acc[mm][4]) | (bf16_rne(acc[mm][5]) << 16),
                          bf16_rne(acc[mm][6]) | (bf16_rne(acc[mm][7]) << 16)},
                    reinterpret_cast<u32x4 *>(out));
            if (a1)
                __builtin_nontemporal_store(
                    u32x4{bf16_rne(acc[mm][8]) | (bf16_rne(acc[mm][9]) << 16),
                          bf16_rne(acc[mm][10]) | (bf16_rne(acc[mm][11]) << 16),
                          bf16_rne(acc[mm][12]) | (bf16_rne(acc[mm][13]) << 16),
                          bf16_rne(acc[mm][14]) | (bf16_rne(acc[mm][15]) << 16)},
                    reinterpret_cast<u32x4 *>(out + 512));
        }
    }
}

// ---------------------------------------------------------------------------
// copy
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_copy(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Workgroup b records the unit it runs on: XCC_ID (hardware register 20) and
// the shader engine / array / CU fields of HW_ID (register 4, bits 8..15),
// then sleeps so the launch cannot finish on a few units.
__global__ __launch_bounds__(64) void k_cu_census(uint32_t *__restrict__ ids, int naps) {
    if (threadIdx.x == 0) {
        const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
        const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u;
        ids[blockIdx.x] = (xcc << 16) | ((hw >> 8) & 0xFFu);
    }
    for (int i = 0; i < naps; ++i) __builtin_amdgcn_s_sleep(127);
}

}  // namespace

hipError_t launch_layout(const LayoutArgs &a, hipStream_t s) {
    const size_t lds = layout_lds_bytes(a.E + a.R);
    // one tile: up to kLayoutReplicas copies, each writing a slice of the
    // outputs; several: the tiles and the src_expert_off block
    const int grid = a.num_tiles > 1 ? a.num_tiles + 1 : max(1, min(a.R, kLayoutReplicas));
    if (a.k <= 8)
        hipLaunchKernelGGL(k_layout<8>, dim3(grid), dim3(kTileTokens), lds, s, a);
    else
        hipLaunchKernelGGL(k_layout<kMaxTopk>, dim3(grid), dim3(kTileTokens), lds, s, a);
    return hipGetLastError();
}

template <int KMAX, bool FP8>
const void *layout_dispatch_kernel(int mode) {
    return mode == kRowsPerRank ? (const void *)k_layout_dispatch<KMAX, FP8, kRowsPerRank>
                                : (const void *)k_layout_dispatch<KMAX, FP8, kRowsPerExpert>;
}

const void *layout_dispatch_fn(int k, bool fp8, int mode) {
    if (k <= 8) return fp8 ? layout_dispatch_kernel<8, true>(mode) : layout_dispatch_kernel<8, false>(mode);
    return fp8 ? layout_dispatch_kernel<kMaxTopk, true>(mode) : layout_dispatch_kernel<kMaxTopk, false>(mode);
}

int layout_dispatch_blocks_per_cu(int k, bool fp8, int mode, size_t lds) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, layout_dispatch_fn(k, fp8, mode), kTileTokens, lds) !=
        hipSuccess)
        return 0;
    return n;
}

template <int KMAX, bool FP8>
void launch_layout_dispatch_t(const LayoutArgs &la, const DispatchArgs &da, int mode, dim3 grid, size_t lds,
                              int lgrid, int extra, hipStream_t s) {
    if (mode == kRowsPerRank)
        hipLaunchKernelGGL((k_layout_dispatch<KMAX, FP8, kRowsPerRank>), grid, dim3(kTileTokens), lds, s, la, da,
                           lgrid, extra);
    else
        hipLaunchKernelGGL((k_layout_dispatch<KMAX, FP8, kRowsPerExpert>), grid, dim3(kTileTokens), lds, s, la, da,
                           lgrid, extra);
}

hipError_t launch_layout_dispatch(const LayoutArgs &la, const DispatchArgs &da, bool fp8, int mode, int num_waves,
                                  int resident_blocks, hipStream_t s) {
    const size_t lds = layout_lds_bytes(la.E + la.R);
    const int lgrid = la.num_tiles > 1 ? la.num_tiles : max(1, min(la.R, kLayoutReplicas));
    // items the layout blocks' waves take: the overflow of a grid that would
    // not be resident at once, if the layout blocks all are
    int extra = 0;
    const int full = lgrid + (num_waves + kWavesPerBlock - 1) / kWavesPerBlock;
    if (!la.use_ticket && resident_blocks > 0 && full > resident_blocks)
        extra = min(num_waves, min(lgrid, full - resident_blocks) * kWavesPerBlock);
    // (several tiles: one more block, last, writes src_expert_off)
    const dim3 grid(lgrid + (num_waves - extra + kWavesPerBlock - 1) / kWavesPerBlock + (la.num_tiles > 1 ? 1 : 0));
    if (la.k <= 8) {
        if (fp8)
            launch_layout_dispatch_t<8, true>(la, da, mode, grid, lds, lgrid, extra, s);
        else
            launch_layout_dispatch_t<8, false>(la, da, mode, grid, lds, lgrid, extra, s);
    } else {
        if (fp8)
            launch_layout_dispatch_t<kMaxTopk, true>(la, da, mode, grid, lds, lgrid, extra, s);
        else
            launch_layout_dispatch_t<kMaxTopk, false>(la, da, mode, grid, lds, lgrid, extra, s);
    }
    return hipGetLastError();
}

hipError_t launch_dispatch_inblock(const LayoutArgs &la, const DispatchArgs &da, bool fp8, int num_waves,
                                   hipStream_t s) {
    const size_t lds = inblock_lds_bytes(la.E + la.R, la.k);
    const dim3 grid((num_waves + kWavesPerBlock - 1) / kWavesPerBlock), block(kTileTokens);
    // row loads per wave fixed at compile time, as in the low-latency kernel
    const int ppw = da.passes_per_wave;
    const int sel = (la.k <= 8 ? 0 : 4) + (fp8 ? 0 : 8) + (ppw <= 1 ? 0 : ppw <= 2 ? 1 : ppw <= 4 ? 2 : 3);
    static void (*const kernels[16])(LayoutArgs, DispatchArgs) = {
        k_dispatch_inblock<8, true, 1>,         k_dispatch_inblock<8, true, 2>,
        k_dispatch_inblock<8, true, 4>,         k_dispatch_inblock<8, true, 8>,
        k_dispatch_inblock<kMaxTopk, true, 1>,  k_dispatch_inblock<kMaxTopk, true, 2>,
        k_dispatch_inblock<kMaxTopk, true, 4>,  k_dispatch_inblock<kMaxTopk, true, 8>,
        k_dispatch_inblock<8, false, 1>,        k_dispatch_inblock<8, false, 2>,
        k_dispatch_inblock<8, false, 4>,        k_dispatch_inblock<8, false, 8>,
        k_dispatch_inblock<kMaxTopk, false, 1>, k_dispatch_inblock<kMaxTopk, false, 2>,
        k_dispatch_inblock<kMaxTopk, false, 4>, k_dispatch_inblock<kMaxTopk, false, 8>};
    hipLaunchKernelGGL(kernels[sel], grid, block, lds, s, la, da);
    return hipGetLastError();
}

template <int MODE>
void launch_dispatch_t(const DispatchArgs &a, bool fp8, dim3 grid, dim3 block, hipStream_t s) {
    if (fp8)
        hipLaunchKernelGGL((k_dispatch<true, MODE>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_dispatch<false, MODE>), grid, block, 0, s, a);
}

hipError_t launch_dispatch(const DispatchArgs &a, bool fp8, int mode, int num_waves, hipStream_t s) {
    const dim3 grid((num_waves + kWavesPerBlock - 1) / kWavesPerBlock), block(kWavesPerBlock * 64);
    if (mode == kRowsPerExpert)
        launch_dispatch_t<kRowsPerExpert>(a, fp8, grid, block, s);
    else if (mode == kRowsPerRank)
        launch_dispatch_t<kRowsPerRank>(a, fp8, grid, block, s);
    else
        launch_dispatch_t<kRowsFromHandle>(a, fp8, grid, block, s);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs &a, bool out_f32, bool prereduce, int num_waves, int cus,
                          hipStream_t s) {
    if (prereduce) {
        // M received rows per wave (M * k lanes hold their routing entries),
        // expert outputs loaded C pairs at a time. At 4096 tokens x 7168,
        // top-8, 32 ranks (28153 rows) on MI355X: M = 4, C = 8 146.5 us;
        // C = 4 149.2; M = 2 154.1; M = 8 169.2; M = 1 246.0 (same GPU).
        constexpr int kPreM = 4, kPreC = 8;
        const int m = a.k <= 16 ? 4 : a.k <= 32 ? 2 : 1;
        const int waves = (int)((a.T + m - 1) / m) * a.npass;
        const dim3 grid((waves + kWavesPerBlock - 1) / kWavesPerBlock), block(kWavesPerBlock * 64);
        void (*fn)(CombineArgs) =
            m == kPreM ? (out_f32 ? k_prereduce<true, kPreM, kPreC> : k_prereduce<false, kPreM, kPreC>)
            : m == 2   ? (out_f32 ? k_prereduce<true, 2, kPreC> : k_prereduce<false, 2, kPreC>)
                       : (out_f32 ? k_prereduce<true, 1, kPreC> : k_prereduce<false, 1, kPreC>);
        hipLaunchKernelGGL(fn, grid, block, 0, s, a);
        return hipGetLastError();
    }
    // A long combine runs at most 8 waves per CU, in two-wave workgroups
    // that each reserve LDS they do not use, so that fewer tokens' rows are
    // read at once. Those reads then fall in a narrower window of the expert
    // outputs, which the DRAM serves faster. Measured on MI355X, 4096 tokens
    // x 7168 top-8 (112 waves per CU): 88.2-89.8 us with four-wave
    // workgroups, 2 per CU, against 91.2-91.5 us uncapped (prefill step 150.7
    // against 153.8 us), and 88.0 against 89.1 us with two-wave workgroups;
    // 16384 tokens (BF16): 348.8-352.2 against 375.8 us. 4, 6 and 12 waves
    // per CU gain less or lose. Shorter combines lose by the cap (1024
    // tokens: 24.9 against 23.4 us; 2048: 46.3 against 45.6), so it starts
    // at 64 waves per CU.
    if (cus > 0 && num_waves >= kCombineCapMinWavesPerCu * cus) {
        const dim3 grid((num_waves + 1) / 2), block(2 * 64);
        hipLaunchKernelGGL((out_f32 ? k_combine<true, 2> : k_combine<false, 2>), grid, block, kCombineCapLds, s, a);
        return hipGetLastError();
    }
    const dim3 grid((num_waves + kWavesPerBlock - 1) / kWavesPerBlock), block(kWavesPerBlock * 64);
    hipLaunchKernelGGL((out_f32 ? k_combine<true, kWavesPerBlock> : k_combine<false, kWavesPerBlock>), grid, block,
                       0, s, a);
    return hipGetLastError();
}

hipError_t launch_cu_census(int blocks, int naps, uint32_t *ids, hipStream_t s) {
    hipLaunchKernelGGL(k_cu_census, dim3(blocks), dim3(64), 0, s, ids, naps);
    return hipGetLastError();
}

size_t ll_lds_bytes(int E, int k, int tpr) { return (size_t)((tpr + 63) / 64) * E * 8 + (size_t)tpr * k * 4; }

hipError_t launch_ll_dispatch(const DispatchArgs &a, bool fp8, int R, int32_t *recv_count, hipStream_t s) {
    const int tpr = a.T / R;
    const int bps = (tpr * a.waves_per_token + kWavesPerBlock - 1) / kWavesPerBlock;
    const dim3 grid(max(R * bps, 1)), block(kTileTokens);
    const size_t lds = ll_lds_bytes(a.E, a.k, tpr);
    // row loads per wave fixed at compile time: 1, 2, 4 or 8 passes (at
    // least the wave's own; at 128 tokens x 7168 each wave holds one pass,
    // and issuing the 14 loads of the 7 passes it does not hold cost 0.4 us
    // per step on MI355X)
    const int ppw = a.passes_per_wave;
    const int sel = (a.k <= 8 ? 0 : 4) + (fp8 ? 0 : 8) + (ppw <= 1 ? 0 : ppw <= 2 ? 1 : ppw <= 4 ? 2 : 3);
    static void (*const kernels[16])(DispatchArgs, int, int, int, int32_t *) = {
        k_ll_dispatch<8, true, 1>,          k_ll_dispatch<8, true, 2>,
        k_ll_dispatch<8, true, 4>,          k_ll_dispatch<8, true, 8>,
        k_ll_dispatch<kMaxTopk, true, 1>,   k_ll_dispatch<kMaxTopk, true, 2>,
        k_ll_dispatch<kMaxTopk, true, 4>,   k_ll_dispatch<kMaxTopk, true, 8>,
        k_ll_dispatch<8, false, 1>,         k_ll_dispatch<8, false, 2>,
        k_ll_dispatch<8, false, 4>,         k_ll_dispatch<8, false, 8>,
        k_ll_dispatch<kMaxTopk, false, 1>,  k_ll_dispatch<kMaxTopk, false, 2>,
        k_ll_dispatch<kMaxTopk, false, 4>,  k_ll_dispatch<kMaxTopk, false, 8>};
    hipLaunchKernelGGL(kernels[sel], grid, block, lds, s, a, R, tpr, bps, recv_count);
    return hipGetLastError();
}

hipError_t launch_copy(const void *src, void *dst, size_t n16, hipStream_t s) {
    const size_t want = (n16 + 255) / 256;
    const unsigned blocks = (unsigned)(want < 256 * 64 ? (want ? want : 1) : 256 * 64);
    hipLaunchKernelGGL(k_copy, dim3(blocks), dim3(256), 0, s, static_cast<const u32x4 *>(src),
                       static_cast<u32x4 *>(dst), n16);
    return hipGetLastError();
}

}  // namespace ep
