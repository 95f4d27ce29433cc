// ltopk_kernels.hip -- top-k index selection for CSA on MI355X (gfx950, wave64).
//
// The selection (per row: the first min(k, |V|) valid positions by score,
// highest first, lower index first among equal scores) is the indexer top-k
// of DeepSeek-V4's compressed sparse attention: k = 512 per index-source layer,
// 2048 eight-position blocks for the shared-candidate layer ("SGLang 与 Miles 为
// DeepSeek-V4.1 提供首日支持", xhh.club, Q&A on cross-layer sharing). The talk
// notes on devpress.csdn.net (section 3.2) time it at a 1M-token context, batch
// size 1, and the AICon 2026 Shenzhen speaker page (aicon.infoq.cn, outline
// 三.2) describes their kernel as per-block histograms of a sharded row merged
// inside a thread-block cluster. CDNA4 has no clusters, LDS is private to a
// workgroup and every dependent device-scope round trip costs about a
// microsecond, so this file avoids histogram merging altogether (below).
//
// Common machinery (own design):
//   * every score becomes an order-preserving 32-bit key (integer ops only);
//     key 0 marks "no element", NaN maps to 1, -0.0 maps to +0.0's key;
//   * the pair (key, ~index) is a 64-bit composite that is unique per
//     position, so "the m largest composites" is exactly the selection rule,
//     ties included, whatever order elements are visited in;
//   * an MSB-first radix select over the composite (digits of 12/10/10 or
//     11/11/10 bits over the key, then 11/11/10 over the inverted index) ends
//     at a prefix P of depth D such that the elements whose D-digit prefix is
//     >= P are exactly the m selected ones; most rows stop after one or two
//     key digits;
//   * digit histograms live in LDS; wave scans use DPP row shifts and row
//     broadcasts instead of LDS permutes.
//
// Kernels:
//   split_kernel  : one row over S workgroups, keys in VGPRs. With S == 1 the
//                   workgroup selects exactly. With S > 1 each workgroup
//                   publishes, without waiting for anyone, every element at or
//                   above a bound B_g chosen so that at least r of its
//                   elements qualify (r covers its expected share of the row's
//                   top-m many standard deviations over); the last workgroup
//                   to finish (ticket counter) selects the top-m of the union
//                   and checks that no workgroup could hold an unpublished
//                   element that belongs in it (B_g <= the m-th composite for
//                   every truncated workgroup). If the check fails -- only for
//                   rows whose best scores cluster in a few chunks -- the same
//                   workgroup re-reads those chunks and selects exactly. One
//                   exchange, no inter-workgroup wait, no co-residency needed.
//                   Plain rows over 2..64 workgroups also have a second mode,
//                   chosen per row record by the previous call: every
//                   workgroup reads the same sample of the whole row (64
//                   scores per chunk), takes the same threshold from it and
//                   the same region sizes from its per-chunk counts, and
//                   publishes every score at or above the threshold -- no
//                   second pass when the winners cluster. For plain rows of
//                   four scores per thread the gathered slots are in index
//                   order, so ties on the last key are broken by slot order
//                   (one prefix over ballot counts) instead of index digits.
//                   Batch size 1, the block / candidate stages.
//   stream_kernel : one wave per row reads the row once from HBM with
//                   non-temporal 16-byte loads kept several sweeps in flight,
//                   admits only scores above the running k-th best (about four
//                   integer ops per score), buffers them in LDS and compacts
//                   by radix select when the buffer fills. Causal prefill.
//   row_kernel    : one 1024-thread workgroup per whole row of up to 32,768
//                   scores, no exchange: a bound from per-thread maxima, the
//                   scores at or above it marked, compacted through LDS and
//                   selected exactly in registers. Decode batches.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "ltopk.h"
#include "ltopk_debug.h"

namespace ltk {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kCapF = 8064;         // candidates the last workgroup of a split row gathers
constexpr int kMaxS = 1024;         // workgroups per split row
constexpr int kMaxSplitRows = 1024; // rows whose workspace one launch may need

// ------------------------------------------------------------------ keys

// Order-preserving map from fp32 bits to an unsigned key: a larger key is a
// higher score. -0.0 gets +0.0's key, every NaN gets 1 (below -inf, whose key
// is 0x007FFFFF), and 0 is left free to mean "no element".
__device__ __forceinline__ uint32_t score_key(uint32_t u)
{
    uint32_t flip = (uint32_t)((int32_t)u >> 31) | 0x80000000u;
    uint32_t key = u ^ flip;
    key = (u == 0x80000000u) ? 0x80000000u : key;
    key = ((u & 0x7fffffffu) > 0x7f800000u) ? 1u : key;
    return key;
}

// The same map without the -0.0 and NaN fix-ups. It differs from score_key
// only on -0.0 (0x7FFFFFFF instead of 0x80000000) and on NaNs. Against a
// threshold that is itself a score_key value t >= 1 (never 0x7FFFFFFF),
// raw_key(u) > t holds whenever score_key(u) > t, so it can pre-filter.
__device__ __forceinline__ uint32_t raw_key(uint32_t u)
{
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ uint64_t comp(uint32_t key, uint32_t nid)
{
    return ((uint64_t)key << 32) | nid;
}

// Prefix of a composite: its bits at and above `s` (s == 64: empty prefix).
__device__ __forceinline__ uint64_t pfx(uint64_t c, int s)
{
    return s >= 64 ? 0ull : (c >> s);
}

// Where a radix select stands. Elements are compared through their prefix
// pfx(c, s): those whose prefix is > P are selected (`above` of them), `cnt`
// have prefix == P and `need` of those still have to be taken. Exact when
// cnt == need: the selection is then every element with pfx(c, s) >= P. Each
// pass fixes the next W bits below s (W <= the histogram's width), so a
// select may start at any s -- right below the bits all its elements share.
struct SelState {
    int s;
    uint64_t P;
    uint32_t above;
    uint32_t cnt;
    uint32_t need;
};

__device__ __forceinline__ SelState sel_start(uint32_t cnt, uint32_t need)
{
    SelState st;
    st.s = 64;
    st.P = 0;
    st.above = 0;
    st.cnt = cnt;
    st.need = need;
    return st;
}

// Start below the common prefix of all elements, known to lie in [lo, hi].
__device__ __forceinline__ SelState sel_start_range(uint64_t lo, uint64_t hi, uint32_t cnt,
                                                    uint32_t need)
{
    SelState st = sel_start(cnt, need);
    const uint64_t d = lo ^ hi;
    st.s = d == 0ull ? 0 : 64 - (int)__builtin_clzll(d);
    st.P = pfx(lo, st.s);
    return st;
}

__device__ __forceinline__ int sel_width(const SelState &st, int maxw)
{
    return st.s < maxw ? st.s : maxw;
}

// Smallest composite whose prefix is P: the selection's lower edge.
__device__ __forceinline__ uint64_t sel_floor(const SelState &st)
{
    return st.s >= 64 ? 0ull : (st.P << st.s);
}

struct BinHit {
    uint32_t bin, above, count, total;
};

__device__ __forceinline__ void advance(SelState &st, const BinHit &h, int W)
{
    st.above += h.above;
    st.need -= h.above;
    st.P = (st.s >= 64 ? 0ull : (st.P << W)) | h.bin;
    st.cnt = h.count;
    st.s -= W;
}

// ---------------------------------------------------------- wave primitives

// DPP move from another lane; lanes with no source (or masked rows) get `id`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp(uint32_t v, uint32_t id)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROWS, 0xf, false);
}

// Inclusive prefix sum across the 64 lanes: Kogge-Stone inside each row of 16
// lanes (row_shr 1, 2, 4, 8), then the row totals are carried with
// row_bcast:15 (into rows 1 and 3) and row_bcast:31 (into rows 2 and 3).
__device__ __forceinline__ uint32_t wave_incl_prefix(uint32_t v)
{
    v += dpp<0x111, 0xf>(v, 0u);
    v += dpp<0x112, 0xf>(v, 0u);
    v += dpp<0x114, 0xf>(v, 0u);
    v += dpp<0x118, 0xf>(v, 0u);
    v += dpp<0x142, 0xa>(v, 0u);
    v += dpp<0x143, 0xc>(v, 0u);
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp<0x111, 0xf>(v, 0u));
    v = max(v, dpp<0x112, 0xf>(v, 0u));
    v = max(v, dpp<0x114, 0xf>(v, 0u));
    v = max(v, dpp<0x118, 0xf>(v, 0u));
    v = max(v, dpp<0x142, 0xa>(v, 0u));
    v = max(v, dpp<0x143, 0xc>(v, 0u));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    v = min(v, dpp<0x111, 0xf>(v, 0xffffffffu));
    v = min(v, dpp<0x112, 0xf>(v, 0xffffffffu));
    v = min(v, dpp<0x114, 0xf>(v, 0xffffffffu));
    v = min(v, dpp<0x118, 0xf>(v, 0xffffffffu));
    v = min(v, dpp<0x142, 0xa>(v, 0xffffffffu));
    v = min(v, dpp<0x143, 0xc>(v, 0xffffffffu));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Smallest 64-bit composite over the wave (~0 for lanes passing ~0).
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v)
{
    const uint32_t hi = wave_min_u32((uint32_t)(v >> 32));
    const uint32_t lo = wave_min_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0xffffffffu);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
    const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
    return ((uint64_t)hi << 32) | lo;
}

// A value every lane holds alike, marked so for the compiler (kept in a scalar
// register, so branches on it need no lane masks).
__device__ __forceinline__ uint32_t uni(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ __forceinline__ uint32_t lane_rank(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Orders this wave's LDS accesses (the only agents touching a single-wave
// workgroup's LDS) and stops the compiler from moving them across.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Threshold bin from an LDS histogram held by one wave: lane l owns the
// nbins/64 bins just below nbins - l*per, so bins above a lane's own belong to
// lower lanes and a prefix sum over lanes gives the count above. Valid only if
// total >= need >= 1.
__device__ __forceinline__ BinHit wave_find_bin(const uint32_t *hist, int nbins, uint32_t need)
{
    const int lane = threadIdx.x & 63;
    const int per = nbins >> 6;
    const int hi = nbins - lane * per;
    const int lo = hi - per;
    uint32_t s = 0;
    for (int b = lo; b < hi; b += 4) {
        const uint4 q = *reinterpret_cast<const uint4 *>(hist + b);
        s += q.x + q.y + q.z + q.w;
    }
    const uint32_t inc = wave_incl_prefix(s);
    const uint32_t above = inc - s;
    const bool mine = s > 0 && above < need && above + s >= need;
    uint32_t bin = 0, run = above, cnt = 0;
    if (mine) {
        for (int b = hi - 1; b >= lo; --b) {
            const uint32_t h = hist[b];
            if (run + h >= need) {
                bin = (uint32_t)b;
                cnt = h;
                break;
            }
            run += h;
        }
    }
    const uint64_t m = __ballot(mine);
    const int src = m ? (int)__builtin_ctzll(m) : 0;
    BinHit r;
    r.bin = (uint32_t)__builtin_amdgcn_readlane((int)bin, src);
    r.above = (uint32_t)__builtin_amdgcn_readlane((int)run, src);
    r.count = (uint32_t)__builtin_amdgcn_readlane((int)cnt, src);
    r.total = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    return r;
}

// Radix select by one wave over n composites in LDS (key 0 = empty slot),
// continued from st until exact or -- with limit > 0 -- until the elements at
// or above the prefix number at most `limit`. hist holds 1 << MAXW words.
template <int MAXW>
__device__ void wave_lds_select(const uint32_t *ckey, const uint32_t *cnid, uint32_t n,
                                SelState &st, uint32_t *hist, uint32_t limit = 0u)
{
    const int lane = threadIdx.x & 63;
    while (st.cnt != st.need && st.s > 0 && (limit == 0u || st.above + st.cnt > limit)) {
        const int W = sel_width(st, MAXW);
        const int sd = st.s - W;
        const int nb = 1 << W;
        const int nz = nb < 256 ? 256 : nb;
        for (int b = lane * 4; b < nz; b += 256)
            *reinterpret_cast<uint4 *>(hist + b) = make_uint4(0u, 0u, 0u, 0u);
        wave_sync();
        // eight entries per lane per step: their LDS reads overlap
        for (uint32_t i0 = 0; i0 < n; i0 += 512) {
            uint32_t kk[8], nn[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t i = i0 + q * 64 + lane;
                kk[q] = i < n ? ckey[i] : 0u;
                nn[q] = i < n ? cnid[i] : 0u;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint64_t c = comp(kk[q], nn[q]);
                if (kk[q] != 0u && pfx(c, st.s) == st.P)
                    atomicAdd(&hist[(uint32_t)(c >> sd) & (uint32_t)(nb - 1)], 1u);
            }
        }
        wave_sync();
        const BinHit h = wave_find_bin(hist, nz, st.need);
        wave_sync();
        if (h.total < st.need)
            break;
        advance(st, h, W);
    }
}

// ---------------------------------------------------------- block primitives

// Exclusive prefix sum of v over the block in thread order; total over all.
// tmp: LDS scratch of T/64 words. With TAIL_SYNC false the closing barrier
// (which guards tmp against the next writer) is left to the caller.
template <int T, bool TAIL_SYNC = true>
__device__ __forceinline__ uint32_t block_excl_prefix(uint32_t v, uint32_t *tmp, uint32_t &total)
{
    constexpr int NW = T / 64;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const uint32_t inc = wave_incl_prefix(v);
    if (lane == 63)
        tmp[w] = inc;
    __syncthreads();
    // the wave totals are combined across lanes (one read per lane), not by
    // every thread looping over them
    const uint32_t part = lane < NW ? tmp[lane] : 0u;
    const uint32_t pinc = wave_incl_prefix(part);
    const uint32_t off = (uint32_t)__builtin_amdgcn_readlane((int)(pinc - part), w);
    total = (uint32_t)__builtin_amdgcn_readlane((int)pinc, 63);
    if (TAIL_SYNC)
        __syncthreads();
    return off + inc - v;
}

// Block-wide threshold bin of an LDS histogram (nbins >= T, powers of two).
// Thread t owns the nbins/T bins just below nbins - t*per, so the count above
// a thread's bins is an exclusive prefix sum over threads.
template <int T>
__device__ __forceinline__ BinHit block_find_bin(const uint32_t *hist, int nbins, uint32_t need,
                                                 uint32_t *tmp, uint32_t *res)
{
    constexpr int NW = T / 64;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int per = nbins / T;
    const int hi = nbins - (int)threadIdx.x * per;
    const int lo = hi - per;
    uint32_t s = 0;
    uint4 q4 = {0u, 0u, 0u, 0u}; // per == 4: the thread's bins, kept for the search below
    if (per == 4) {
        q4 = *reinterpret_cast<const uint4 *>(hist + lo);
        s = q4.x + q4.y + q4.z + q4.w;
    } else if (per > 4) {
        for (int b = lo; b < hi; b += 4) {
            const uint4 q = *reinterpret_cast<const uint4 *>(hist + b);
            s += q.x + q.y + q.z + q.w;
        }
    } else {
        for (int b = lo; b < hi; ++b)
            s += hist[b];
    }
    const uint32_t inc = wave_incl_prefix(s);
    if ((threadIdx.x & 63) == 63)
        tmp[w] = inc;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const uint32_t part = lane < NW ? tmp[lane] : 0u;
    const uint32_t pinc = wave_incl_prefix(part);
    const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(pinc - part), w) + inc - s;
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)pinc, 63);
    if (s > 0 && above < need && above + s >= need) {
        if (per == 4) {
            // from the top bin (hi - 1, the vector's last word) down
            const uint32_t r3 = above, r2 = r3 + q4.w, r1 = r2 + q4.z, r0 = r1 + q4.y;
            const int d = r2 >= need ? 3 : r1 >= need ? 2 : r0 >= need ? 1 : 0;
            res[0] = (uint32_t)(lo + d);
            res[1] = d == 3 ? r3 : d == 2 ? r2 : d == 1 ? r1 : r0;
            res[2] = d == 3 ? q4.w : d == 2 ? q4.z : d == 1 ? q4.y : q4.x;
        } else if (per == 1) {
            res[0] = (uint32_t)lo;
            res[1] = above;
            res[2] = s;
        } else {
            uint32_t run = above;
            for (int b = hi - 1; b >= lo; --b) {
                const uint32_t h = hist[b];
                if (run + h >= need) {
                    res[0] = (uint32_t)b;
                    res[1] = run;
                    res[2] = h;
                    break;
                }
                run += h;
            }
        }
    }
    __syncthreads();
    BinHit r;
    r.bin = (uint32_t)__builtin_amdgcn_readfirstlane((int)res[0]);
    r.above = (uint32_t)__builtin_amdgcn_readfirstlane((int)res[1]);
    r.count = (uint32_t)__builtin_amdgcn_readfirstlane((int)res[2]);
    r.total = (uint32_t)__builtin_amdgcn_readfirstlane((int)total);
    return r;
}

template <int T>
__device__ __forceinline__ void block_zero(uint32_t *a, int n)
{
    for (int i = (int)threadIdx.x * 4; i < n; i += T * 4)
        *reinterpret_cast<uint4 *>(a + i) = make_uint4(0u, 0u, 0u, 0u);
}

// ------------------------------------------------------------------ params

enum Mode { MODE_PLAIN = 0, MODE_BLOCKS = 1, MODE_CAND = 2 };

// A zero word read in place of a row's mode word by launches that do not
// sample (never written).
static __device__ uint32_t g_zero_word;

struct KParams {
    const float *scores;
    int64_t row_stride;
    const int32_t *lengths;
    int32_t n_max;
    int32_t k;           // k, or kb for the block stage
    const int32_t *cand; // [B, n_cand] block ids (MODE_CAND)
    int32_t n_cand;
    int32_t bs;          // block size (MODE_BLOCKS, MODE_CAND)
    int32_t row0;        // first row of this launch
    int32_t *out;        // [B, k]
    uint32_t *ws;        // workspace (split rows with S > 1)
    int64_t vlen;        // length of the virtual row (positions, blocks or slots)
    uint32_t force_fallback;
    uint32_t force_sample; // 0 the mode word decides, 1 never sample, 2 always
};

// Per-row workspace (32-bit words): counters, one 16-byte record per
// workgroup (valid count, truncated flag, bound B_g), and the candidate
// regions as (key, ~index) pairs.
constexpr int kWsTicket = 0;
constexpr int kWsMode = 1; // split rows that may sample: 1 = take the sampled threshold
constexpr int kWsMeta = 64;
constexpr int kWsRegion = kWsMeta + 4 * kMaxS;
constexpr int kWsRowWords = kWsRegion + 2 * kCapF; // 20288 words = 81152 bytes

__device__ __forceinline__ int32_t row_len(const KParams &p, int row)
{
    int32_t len = p.lengths[row];
    return len < 0 ? 0 : (len > p.n_max ? p.n_max : len);
}

// Valid elements of the virtual row (positions, blocks, or candidate slots:
// for candidates this is an upper bound, the exact count comes from the keys).
__device__ __forceinline__ int64_t virtual_len(const KParams &p, int MODE_, int32_t len)
{
    if (MODE_ == MODE_BLOCKS)
        return (len + (int64_t)p.bs - 1) / p.bs;
    if (MODE_ == MODE_CAND)
        return p.vlen;
    return len;
}

// ------------------------------------------------------------------ loaders

// Buffer resource over the scores of [base, len) of a row (bytes past len
// read as zero without touching memory). Buffer loads are not ordinary IR
// loads, so the compiler neither merges them across loop iterations nor puts
// them behind branches, and every load of a chunk can be in flight at once.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float *x, int64_t base, int64_t len)
{
    const int64_t rem = len > base ? (len - base) * 4 : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void *)(x + base), (short)0,
                                             (int)(rem < 0x7ffffff0 ? rem : 0x7ffffff0),
                                             0x00020000);
}

__device__ __forceinline__ u4 load16(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)byte_off, 0, 0);
}

// Streaming variant: the non-temporal hint lets the caches drop lines that
// are read exactly once.
__device__ __forceinline__ u4 load16_nt(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)byte_off, 0, 2);
}

// Fill key[E] / nid[E] (nid = ~position) for this thread's share of the
// chunk of the virtual row starting at `base`. Absent elements get key 0.
template <int T, int E, int MODE>
struct Loader;

template <int T, int E>
struct Loader<T, E, MODE_PLAIN> {
    static_assert(E % 4 == 0, "plain rows load 4 scores per vector");
    static __device__ __forceinline__ void load(const KParams &p, int row, int32_t len, int64_t base,
                                                uint32_t (&key)[E], uint32_t (&nid)[E])
    {
        const float *x = p.scores + (int64_t)row * p.row_stride;
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(x, base, len);
        u4 f[E / 4];
#pragma unroll
        for (int g = 0; g < E / 4; ++g)
            f[g] = load16(rs, (uint32_t)(g * T + threadIdx.x) * 16u);
#pragma unroll
        for (int g = 0; g < E / 4; ++g) {
            const int64_t v0 = base + ((int64_t)g * T + threadIdx.x) * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t i = v0 + j;
                key[4 * g + j] = (i < len) ? score_key(f[g][j]) : 0u;
                nid[4 * g + j] = ~(uint32_t)i;
            }
        }
    }
};

// Virtual element = a block of bs positions scored by its best valid key.
template <int T, int E>
struct Loader<T, E, MODE_BLOCKS> {
    static __device__ __forceinline__ void load(const KParams &p, int row, int32_t len, int64_t base,
                                                uint32_t (&key)[E], uint32_t (&nid)[E])
    {
        const float *x = p.scores + (int64_t)row * p.row_stride;
        const int64_t bs = p.bs;
        const int64_t nb = (len + bs - 1) / bs;
        if (bs == 8) {
            const __amdgpu_buffer_rsrc_t rs = row_rsrc(x, base * 8, len);
            u4 a[E], b[E];
#pragma unroll
            for (int g = 0; g < E; ++g) {
                const uint32_t off = (uint32_t)(g * T + threadIdx.x) * 32u;
                a[g] = load16(rs, off);
                b[g] = load16(rs, off + 16u);
            }
#pragma unroll
            for (int g = 0; g < E; ++g) {
                const int64_t blk = base + (int64_t)g * T + threadIdx.x;
                const int64_t lo = blk * 8;
                uint32_t best = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t ka = (lo + j < len) ? score_key(a[g][j]) : 0u;
                    const uint32_t kb = (lo + 4 + j < len) ? score_key(b[g][j]) : 0u;
                    best = ka > best ? ka : best;
                    best = kb > best ? kb : best;
                }
                key[g] = best;
                nid[g] = ~(uint32_t)blk;
            }
            return;
        }
#pragma unroll
        for (int g = 0; g < E; ++g) {
            const int64_t blk = base + (int64_t)g * T + threadIdx.x;
            uint32_t best = 0;
            if (blk < nb) {
                const int64_t lo = blk * bs;
                const int64_t hi = lo + bs < len ? lo + bs : len;
                for (int64_t i = lo; i < hi; ++i) {
                    const uint32_t kk = score_key(__float_as_uint(x[i]));
                    best = kk > best ? kk : best;
                }
            }
            key[g] = best;
            nid[g] = ~(uint32_t)blk;
        }
    }
};

// Virtual element = slot s of the candidate list expanded to positions:
// slot s -> block cand[s / bs], offset s % bs.
template <int T, int E>
struct Loader<T, E, MODE_CAND> {
    static __device__ __forceinline__ void load(const KParams &p, int row, int32_t len, int64_t base,
                                                uint32_t (&key)[E], uint32_t (&nid)[E])
    {
        const float *x = p.scores + (int64_t)row * p.row_stride;
        const int32_t *cl = p.cand + (int64_t)row * p.n_cand;
        const int64_t bs = p.bs;
        if (bs == 8 && E % 8 == 0 && len < (1 << 28)) {
            const __amdgpu_buffer_rsrc_t rs = row_rsrc(x, 0, len);
            int64_t lo[E / 8];
#pragma unroll
            for (int g = 0; g < E / 8; ++g) {
                const int64_t slot = base / 8 + (int64_t)g * T + threadIdx.x;
                const int64_t b = slot < p.n_cand ? (int64_t)cl[slot] : -1;
                lo[g] = (b >= 0 && b * 8 < len) ? b * 8 : -1;
            }
            u4 f0[E / 8], f1[E / 8];
#pragma unroll
            for (int g = 0; g < E / 8; ++g) {
                // an invalid block reads past the range: zeros, no access
                const uint32_t off = lo[g] >= 0 ? (uint32_t)lo[g] * 4u : 0xfffffff0u;
                f0[g] = load16(rs, off);
                f1[g] = load16(rs, off + 16u);
            }
#pragma unroll
            for (int g = 0; g < E / 8; ++g) {
                const bool ok = lo[g] >= 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    key[8 * g + j] = (ok && lo[g] + j < len) ? score_key(f0[g][j]) : 0u;
                    key[8 * g + 4 + j] = (ok && lo[g] + 4 + j < len) ? score_key(f1[g][j]) : 0u;
                    nid[8 * g + j] = ~(uint32_t)(lo[g] + j);
                    nid[8 * g + 4 + j] = ~(uint32_t)(lo[g] + 4 + j);
                }
            }
            return;
        }
#pragma unroll
        for (int g = 0; g < E; ++g) {
            const int64_t v = base + (int64_t)g * T + threadIdx.x;
            const int64_t c = v / bs;
            const int64_t b = c < p.n_cand ? (int64_t)cl[c] : -1;
            const int64_t pos = b * bs + (v - c * bs);
            const bool ok = b >= 0 && pos < len;
            key[g] = ok ? score_key(__float_as_uint(x[pos])) : 0u;
            nid[g] = ~(uint32_t)pos;
        }
    }
};

// Histogram of the next W-bit digit over register-resident elements whose
// prefix matches st.P. hist must be zeroed and the block synchronised.
template <int E>
__device__ __forceinline__ void regs_hist(const uint32_t (&key)[E], const uint32_t (&nid)[E],
                                          const SelState &st, int W, uint32_t *hist)
{
    const int sd = st.s - W;
    const uint32_t mask = (1u << W) - 1u;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const uint64_t c = comp(key[j], nid[j]);
        if (key[j] != 0u && pfx(c, st.s) == st.P)
            atomicAdd(&hist[(uint32_t)(c >> sd) & mask], 1u);
    }
}

// Radix select over register-resident elements by the whole block: per digit
// one LDS histogram, one barrier after it and the two of block_find_bin. The
// histograms rotate through three LDS buffers of NB words, so none needs a
// barrier of its own for zeroing: the buffer a pass zeroes was last read
// before that pass's barrier and is next written two passes later, after
// another barrier. Digits inside the key use 32-bit arithmetic. Once the key
// is resolved, the index bits above `ibits` are skipped: every nid is ~index
// with index < 2^ibits, so those bits are ones. Runs until exact or -- with
// limit > 0 -- until the elements at or above the prefix number at most
// `limit`; with KEY_ONLY it also stops once the key is resolved (s == 32,
// the last key digit narrowed to end there). With TIES (kw: T / 64 LDS
// words) it stops once every element left at the prefix has one key: at
// s <= 32, or, found by each wave's smallest and largest key at the prefix
// that the passes after the first also take, with s set to 32 and P to that
// key -- the order among them is left to the caller.
// Buffers 0 and 1 must be zero, with a barrier between that and the call;
// all three are left dirty.
template <int MAXW>
struct HistBuf {
    static constexpr int NB = 1 << MAXW;
};

template <int T, int MAXW, int E, bool KEY_ONLY = false, bool TIES = false>
__device__ void block_regs_select(const uint32_t (&key)[E], const uint32_t (&nid)[E], SelState &st,
                                  uint32_t limit, uint32_t *hbuf, uint32_t *tmp, uint32_t *res,
                                  int ibits, uint32_t *kw = nullptr)
{
    constexpr int NB = HistBuf<MAXW>::NB;
    static_assert(NB >= 4 * T, "block_find_bin reads four bins per thread");
    int cur = 0;
    const int s_in = st.s; // TIES: passes after the first start below it
    while (st.cnt != st.need && st.s > (KEY_ONLY || TIES ? 32 : 0) &&
           (limit == 0u || st.above + st.cnt > limit)) {
        if (st.s == 32 && ibits < 32) {
            const int sh = 32 - ibits;
            st.P = (st.P << sh) | ((1ull << sh) - 1ull);
            st.s = ibits;
            continue;
        }
        int W = sel_width(st, MAXW);
        if (KEY_ONLY && st.s - W < 32)
            W = st.s - 32;
        const int sd = st.s - W;
        const uint32_t mask = (1u << W) - 1u;
        uint32_t *h = hbuf + cur * NB;
        uint32_t kmn = 0xffffffffu, kmx = 0u;
        if (sd >= 32) {
            const int ks = st.s - 32;
            const uint32_t P32 = (uint32_t)st.P;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const uint32_t kp = ks >= 32 ? 0u : key[j] >> (ks & 31);
                if (key[j] != 0u && kp == P32) {
                    atomicAdd(&h[(key[j] >> (sd - 32)) & mask], 1u);
                    kmn = min(kmn, key[j]);
                    kmx = max(kmx, key[j]);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const uint64_t c = comp(key[j], nid[j]);
                if (key[j] != 0u && pfx(c, st.s) == st.P) {
                    atomicAdd(&h[(uint32_t)(c >> sd) & mask], 1u);
                    kmn = min(kmn, key[j]);
                    kmx = max(kmx, key[j]);
                }
            }
        }
        if constexpr (TIES) {
            // (not in the first pass, which a spread row ends) the wave's
            // elements at the prefix: none (~0, never a key), all of one
            // key K (K) or of several (0)
            if (st.s != s_in) {
                const uint64_t mk = __ballot(kmx != 0u);
                const uint32_t K =
                    mk != 0ull
                        ? (uint32_t)__builtin_amdgcn_readlane((int)kmx, (int)__builtin_ctzll(mk))
                        : 0xffffffffu;
                const bool mixed = __ballot(kmx != 0u && (kmn != K || kmx != K)) != 0ull;
                if ((threadIdx.x & 63) == 0)
                    kw[threadIdx.x >> 6] = mixed ? 0u : K;
            }
        }
        __syncthreads();
        block_zero<T>(hbuf + ((cur + 2) % 3) * NB, NB);
        if constexpr (TIES) {
            if (st.s != s_in) {
                const uint32_t lane = threadIdx.x & 63u;
                const uint32_t v = lane < (uint32_t)(T / 64) ? kw[lane] : 0xffffffffu;
                const uint64_t any = __ballot(v != 0xffffffffu);
                const uint32_t K =
                    any != 0ull
                        ? (uint32_t)__builtin_amdgcn_readlane((int)v, (int)__builtin_ctzll(any))
                        : 0u;
                if (K != 0u && __ballot(v != 0xffffffffu && v != K) == 0ull) {
                    // every element at the prefix has key K (the histogram
                    // just taken is one bin): no digit separates them
                    st.P = K;
                    st.s = 32;
                    break;
                }
            }
        }
        const BinHit hh = block_find_bin<T>(h, NB, st.need, tmp, res);
        if (hh.total < st.need)
            break;
        advance(st, hh, W);
        cur = (cur + 1) % 3;
    }
}

// Is composite (key, nid) at or above the selection floor F (key 0 = absent)?
__device__ __forceinline__ bool at_or_above(uint32_t key, uint32_t nid, uint32_t fk, uint32_t fn)
{
    return key != 0u && (key > fk || (key == fk && nid >= fn));
}

// Bits needed for indices below `bound` (0 when bound <= 1).
__device__ __forceinline__ int index_bits(int64_t bound)
{
    return bound <= 1 ? 0 : 64 - __builtin_clzll((uint64_t)(bound - 1));
}

// Ends a select whose elements left at the prefix (st.s <= 32) all have one
// key K, for G elements per thread held in slot order (slot threadIdx.x + j T)
// whose indices rise with the slot. Of the cnt tied elements the need with
// the smallest indices win: the first need in slot order. Each tied element
// gets its rank from one count per wave and j (a ballot), an exclusive
// prefix over those counts in slot order and its lane's rank in its ballot,
// in place of a pass per index digit; the tied elements ranked need or
// later are dropped (key 0), so the selection is every element left with a
// key >= K and the state ends exact at the lower edge (K, 0). Needs
// cnt > need >= 1; tcnt holds G T / 64 words.
template <int T, int G>
__device__ void tie_floor_slots(uint32_t (&ckey)[G], const uint32_t (&cnid)[G], SelState &st,
                                uint32_t *tcnt)
{
    constexpr int NW = T / 64;
    constexpr uint32_t NC = (uint32_t)(G * NW);
    static_assert(NC <= 128, "two counts per lane");
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t w = uni(threadIdx.x >> 6);
    uint64_t bal[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        bal[j] = __ballot(ckey[j] != 0u && pfx(comp(ckey[j], cnid[j]), st.s) == st.P);
        if (lane == 0u)
            tcnt[(uint32_t)j * NW + w] = (uint32_t)__popcll(bal[j]);
    }
    __syncthreads();
    const uint32_t a = 2u * lane < NC ? tcnt[2u * lane] : 0u;
    const uint32_t b = 2u * lane + 1u < NC ? tcnt[2u * lane + 1u] : 0u;
    const uint32_t inc = wave_incl_prefix(a + b);
    const uint32_t x0 = inc - a - b, x1 = inc - b; // tied elements before entries 2 l, 2 l + 1
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const uint32_t e = (uint32_t)j * NW + w;
        const uint32_t before =
            (uint32_t)__builtin_amdgcn_readlane((int)((e & 1u) ? x1 : x0), (int)(e >> 1));
        if (((bal[j] >> lane) & 1ull) != 0ull && before + lane_rank(bal[j]) >= st.need)
            ckey[j] = 0u;
    }
    // (tcnt is not written again by this workgroup)
    const uint32_t K = (uint32_t)(st.P >> (32 - st.s));
    st.P = (uint64_t)K << 32;
    st.s = 0;
    st.above += st.need;
    st.cnt = 0u;
    st.need = 0u;
}

// Exact selection over a whole virtual row re-read from memory by one block,
// writing out[0, m) (slots via an LDS counter). The fallback of the split
// kernel; correct for any input, one pass over the row per digit.
template <int T, int E, int MODE, int MAXW>
__device__ void block_row_select(const KParams &p, int row, int32_t len, uint32_t V, uint32_t m,
                                 int32_t *out, uint32_t *hist, uint32_t *tmp, uint32_t *res,
                                 uint32_t *ctr)
{
    constexpr int64_t C = (int64_t)T * E;
    const int64_t vlen = virtual_len(p, MODE, len);
    SelState st = sel_start(V, m);
    uint32_t key[E], nid[E];
    while (st.cnt != st.need && st.s > 0) {
        const int W = sel_width(st, MAXW);
        const int nb = 1 << W;
        const int nz = nb < 4 * T ? 4 * T : nb;
        block_zero<T>(hist, nz);
        __syncthreads();
        for (int64_t base = 0; base < vlen; base += C) {
            Loader<T, E, MODE>::load(p, row, len, base, key, nid);
            regs_hist(key, nid, st, W, hist);
        }
        __syncthreads();
        const BinHit h = block_find_bin<T>(hist, nz, st.need, tmp, res);
        if (h.total < st.need)
            break;
        advance(st, h, W);
    }
    if (threadIdx.x == 0)
        *ctr = 0;
    __syncthreads();
    for (int64_t base = 0; base < vlen; base += C) {
        Loader<T, E, MODE>::load(p, row, len, base, key, nid);
#pragma unroll
        for (int j = 0; j < E; ++j) {
            if (m != 0u && key[j] != 0u && pfx(comp(key[j], nid[j]), st.s) >= st.P) {
                const uint32_t q = atomicAdd(ctr, 1u);
                if (q < m)
                    out[q] = (int32_t)~nid[j];
            }
        }
    }
}

// Exact selection over a union: register-resident candidates (ckey/cnid,
// key 0 = none) plus every element of the chunks list[0, nl) (workgroup
// indices), re-read from memory in each pass. `cnt` counts the union's valid
// elements, all of which lie at or below `hi`; at least m of them are at or
// above `lo`, so the select starts below the bits lo and hi share. out[0, m)
// receives the union's top m (slots via `ctr`, zero on entry). The recovery
// of the split kernel when a few workgroups hold more of the row's top-k than
// they published: only their chunks are read again.
template <int T, int E, int MODE, int MAXW, int G>
__device__ void block_part_select(const KParams &p, int row, int32_t len, const uint32_t *list,
                                  uint32_t nl, uint64_t lo, uint64_t hi, uint32_t cnt, uint32_t m,
                                  const uint32_t (&ckey)[G], const uint32_t (&cnid)[G],
                                  int32_t *out, uint32_t *hist, uint32_t *tmp, uint32_t *res,
                                  uint32_t *ctr)
{
    constexpr int64_t C = (int64_t)T * E;
    // a chunk is re-read in the smallest pieces its loader takes, four pieces
    // in flight at a time; a piece past the list reads nothing (an offset
    // past the virtual row: all keys 0)
    constexpr int EP = MODE == MODE_PLAIN ? 4 : (MODE == MODE_BLOCKS ? 1 : 8);
    constexpr int NPC = E / EP; // pieces per chunk
    constexpr int QF = MODE == MODE_CAND ? 1 : 4; // (a candidate piece is 8 slots already)
    static_assert(E % EP == 0, "chunks are whole pieces");
    const uint32_t np = nl * NPC;
    const int64_t past = virtual_len(p, MODE, len);
    auto piece_base = [&](uint32_t q) {
        return q < np ? (int64_t)list[q / NPC] * C + (int64_t)(q % NPC) * T * EP : past;
    };
    SelState st = sel_start_range(lo, hi, cnt, m);
    uint32_t key[QF][EP], nid[QF][EP];
    while (st.cnt != st.need && st.s > 0) {
        const int W = sel_width(st, MAXW);
        const int nb = 1 << W;
        const int nz = nb < 4 * T ? 4 * T : nb;
        block_zero<T>(hist, nz);
        __syncthreads();
        regs_hist(ckey, cnid, st, W, hist);
        for (uint32_t q0 = 0; q0 < np; q0 += QF) {
#pragma unroll
            for (int u = 0; u < QF; ++u)
                Loader<T, EP, MODE>::load(p, row, len, piece_base(q0 + u), key[u], nid[u]);
#pragma unroll
            for (int u = 0; u < QF; ++u)
                regs_hist(key[u], nid[u], st, W, hist);
        }
        __syncthreads();
        const BinHit h = block_find_bin<T>(hist, nz, st.need, tmp, res);
        if (h.total < st.need)
            break;
        advance(st, h, W);
    }
    const uint64_t F = sel_floor(st);
    auto emit = [&](uint32_t kk, uint32_t nn) {
        if (m != 0u && kk != 0u && comp(kk, nn) >= F) {
            const uint32_t q = atomicAdd(ctr, 1u);
            if (q < m)
                out[q] = (int32_t)~nn;
        }
    };
#pragma unroll
    for (int j = 0; j < G; ++j)
        emit(ckey[j], cnid[j]);
    for (uint32_t q0 = 0; q0 < np; q0 += QF) {
#pragma unroll
        for (int u = 0; u < QF; ++u)
            Loader<T, EP, MODE>::load(p, row, len, piece_base(q0 + u), key[u], nid[u]);
#pragma unroll
        for (int u = 0; u < QF; ++u)
#pragma unroll
            for (int j = 0; j < EP; ++j)
                emit(key[u][j], nid[u][j]);
    }
}

// Exact selection over a union that fits LDS: register-resident candidates
// (ckey/cnid, key 0 = none) plus every element of the chunks list[0, nl)
// (workgroup indices), loaded from memory once into `stage`, chunk q at
// [q * C, q * C + C), keys only: an element's index follows from its slot,
// which is why this serves plain rows and blocks (whose index is the virtual
// index) and not candidate lists. At least m of the union's elements are at
// or above `lo`, so the row's top m have keys >= lo's key: elements with a
// smaller key take no part, and the union's elements all lie at or below
// `hi`, so the select starts below the bits lo and hi share.
//
// With 16 waves per workgroup every instruction is paid sixteen times per
// SIMD, so each pass over the staged keys costs microseconds; this makes
// two. The first digit's histogram is taken while staging (h0), and the
// elements at or above the digit's threshold bin (at most 2048) are then
// compacted into per-wave lists (h0: keys, h1: indices, 128 per wave; cw:
// the 16 counts). The select finishes in registers, two elements per thread,
// and out[0, m) receives the union's top m. Returns false, having written no
// output, when the first digit does not lie inside the key or the elements
// left do not fit the lists; the caller then falls back to a selection that
// re-reads the chunks. The recovery of the split kernel when a few
// workgroups hold more of the row's top-k than they published, as long as
// their chunks fit `stage`.
template <int T, int E, int MODE, int MAXW, int G>
__device__ bool staged_part_select(const KParams &p, int row, int32_t len, const uint32_t *list,
                                   uint32_t nl, uint64_t lo, uint64_t hi, uint32_t cnt, uint32_t m,
                                   const uint32_t (&ckey)[G], const uint32_t (&cnid)[G],
                                   int32_t *out, uint32_t *stage, uint32_t *h0, uint32_t *h1,
                                   uint32_t *cw, uint32_t *tmp, uint32_t *res, int ibits)
{
    static_assert(MODE != MODE_CAND, "a candidate slot's index is not its position");
    static_assert(T == 1024, "sixteen per-wave lists");
    constexpr uint32_t C = (uint32_t)T * E;
    static_assert((C & (C - 1)) == 0, "chunks are powers of two");
    constexpr int LOGC = __builtin_ctz(C);
    constexpr int NB = HistBuf<MAXW>::NB;
    constexpr uint32_t RW = 128;     // list slots per wave
    constexpr int SW = (int)RW / 64; // list slots per thread
    const uint32_t ns = nl * C;
    const uint32_t lok = (uint32_t)(lo >> 32);
    const int lane = threadIdx.x & 63;
    const uint32_t wv = uni(threadIdx.x >> 6);

    SelState st = sel_start_range(lo, hi, cnt, m);
    const int W0 = sel_width(st, MAXW);
    if (st.s - W0 < 32)
        return false; // lo and hi share the key's first 21 bits: not this path
    const int ks0 = st.s - 32;
    const uint32_t P0 = (uint32_t)st.P, sh0 = (uint32_t)(st.s - W0 - 32), mask0 = (1u << W0) - 1u;
    auto hit0 = [&](uint32_t kk) {
        return kk >= lok && kk != 0u && (ks0 >= 32 ? 0u : kk >> (ks0 & 31)) == P0;
    };
    block_zero<T>(h0, NB);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < G; ++j)
        if (hit0(ckey[j]))
            atomicAdd(&h0[(ckey[j] >> sh0) & mask0], 1u);
    if constexpr (MODE == MODE_PLAIN) {
        // Raw 16-byte loads of up to CF chunks in flight (a chunk index past
        // the list reads past the row: no memory access), then the key map
        // for the real ones only, written back as 16 bytes per thread and
        // vector (the loader's layout: thread t's vector g covers positions
        // base + (g * T + t) * 4 + [0, 4)).
        constexpr int NV = E / 4;
        constexpr int CF = NV >= 2 ? 1 : 4;
        const float *x = p.scores + (int64_t)row * p.row_stride;
        for (uint32_t q = 0; q < nl; q += CF) {
            u4 f[CF][NV];
#pragma unroll
            for (int u = 0; u < CF; ++u) {
                const int64_t base = (int64_t)(q + u < nl ? list[q + u] : (uint32_t)kMaxS) * C;
                const __amdgpu_buffer_rsrc_t rs = row_rsrc(x, base, len);
#pragma unroll
                for (int g = 0; g < NV; ++g)
                    f[u][g] = load16(rs, (uint32_t)(g * T + threadIdx.x) * 16u);
            }
#pragma unroll
            for (int u = 0; u < CF; ++u) {
                if (q + u < nl) {
                    const int64_t base = (int64_t)list[q + u] * C;
                    const bool tail = base + C > len; // the chunk holding the row's end
#pragma unroll
                    for (int g = 0; g < NV; ++g) {
                        const int64_t i0 = base + ((int64_t)g * T + threadIdx.x) * 4;
                        u4 kv;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            kv[j] = (!tail || i0 + j < len) ? score_key(f[u][g][j]) : 0u;
                        *reinterpret_cast<u4 *>(stage + (q + u) * C +
                                                ((uint32_t)g * T + threadIdx.x) * 4u) = kv;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (hit0(kv[j]))
                                atomicAdd(&h0[(kv[j] >> sh0) & mask0], 1u);
                    }
                }
            }
        }
    } else {
        for (uint32_t q = 0; q < nl; ++q) {
            uint32_t kk[E], nn[E];
            const uint32_t g0 = list[q];
            Loader<T, E, MODE>::load(p, row, len, (int64_t)g0 * C, kk, nn);
#pragma unroll
            for (int j = 0; j < E; ++j) {
                stage[q * C + (~nn[j] - g0 * C)] = kk[j];
                if (hit0(kk[j]))
                    atomicAdd(&h0[(kk[j] >> sh0) & mask0], 1u);
            }
        }
    }
    __syncthreads();
    if (st.cnt != st.need) {
        // (at least m counted elements reach lo, so the bin is always found)
        const BinHit hh = block_find_bin<T>(h0, NB, st.need, tmp, res);
        advance(st, hh, W0);
    }
    if (st.above + st.cnt > 16u * RW)
        return false;

    // ---- the elements at or above the prefix into per-wave lists (h0 was
    // last read by the find-bin, which ended with a barrier)
    const int ks = st.s - 32; // 0 <= ks < 32 here
    const uint32_t P32 = (uint32_t)st.P;
    auto keep = [&](uint32_t kk) { return kk >= lok && kk != 0u && (kk >> ks) >= P32; };
    uint32_t c = 0; // this wave's list length (uniform)
    auto put = [&](bool k, uint32_t kk, uint32_t nn) {
        const uint64_t mk = __ballot(k);
        const uint32_t at = c + lane_rank(mk);
        if (k && at < RW) {
            h0[wv * RW + at] = kk;
            h1[wv * RW + at] = nn;
        }
        c += (uint32_t)__popcll(mk);
    };
#pragma unroll
    for (int j = 0; j < G; ++j)
        put(keep(ckey[j]), ckey[j], cnid[j]);
    // four rows of 64 per step, their reads in flight together; a row's
    // chunk (and so its indices' base) is the same for the whole wave
    for (uint32_t i0 = wv * 64u; i0 < ns; i0 += 4u * T) {
        uint32_t kk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t i = i0 + (uint32_t)u * T + (uint32_t)lane;
            kk[u] = i < ns ? stage[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t r0 = i0 + (uint32_t)u * T; // wave-uniform
            const uint32_t i = r0 + (uint32_t)lane;
            const uint32_t cb = r0 < ns ? uni(list[r0 >> LOGC]) * C - (r0 & ~(C - 1u)) : 0u;
            const bool k = i < ns && keep(kk[u]);
            put(k, kk[u], ~(cb + i));
        }
    }
    if (lane == 0)
        cw[wv] = c;
    __syncthreads();
    if (wave_max_u32(lane < 16 ? cw[lane] : 0u) > RW)
        return false; // (uniform: every wave read the same counts)
    uint32_t sk[SW], sn[SW];
#pragma unroll
    for (int u = 0; u < SW; ++u) {
        const uint32_t at = (uint32_t)lane + (uint32_t)u * 64u;
        sk[u] = at < c ? h0[wv * RW + at] : 0u;
        sn[u] = at < c ? h1[wv * RW + at] : 0u;
    }
    // the staged keys are no longer needed: their space holds the three
    // rotating histograms of the register select
    block_zero<T>(stage, 2 * NB);
    __syncthreads();
    block_regs_select<T, MAXW>(sk, sn, st, 0u, stage, tmp, res, ibits);
    const uint64_t F = sel_floor(st);
    const uint32_t fk = (uint32_t)(F >> 32), fn = (uint32_t)F;
    uint32_t nsel = 0;
#pragma unroll
    for (int u = 0; u < SW; ++u)
        nsel += at_or_above(sk[u], sn[u], fk, fn) ? 1u : 0u;
    uint32_t tot;
    uint32_t q = block_excl_prefix<T>(nsel, tmp, tot);
#pragma unroll
    for (int u = 0; u < SW; ++u) {
        if (at_or_above(sk[u], sn[u], fk, fn)) {
            if (q < m)
                out[q] = (int32_t)~sn[u];
            ++q;
        }
    }
    return true;
}

// ------------------------------------------------------------------ split kernel

// Exchange between the workgroups of a split row. Every word another
// workgroup reads is written with an agent-scope atomic store and read with
// an agent-scope atomic load; on gfx950 these bypass the XCD-local L2 (sc1),
// so the only ordering needed is "my stores are complete before my ticket":
// an explicit wait on the vector-memory counter. A release fence would also
// write back the whole L2 of the XCD, which costs microseconds when dozens of
// workgroups do it at once.
__device__ __forceinline__ void put64(uint64_t *a, uint64_t v)
{
    __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t get64(const uint64_t *a)
{
    return __hip_atomic_load(const_cast<uint64_t *>(a), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wait_stores()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0f70); // vmcnt(0): stores acknowledged
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// WHOLE: the host launches one workgroup per row (S == 1); the code after the
// single-workgroup path is then unreachable, and the kernel needs only that
// path's registers.
// LDS pool of the split kernel's exchange instances (one workgroup per CU
// anyway: they need over 64 VGPRs at 1024 threads). The last workgroup's
// recovery stages flagged chunks behind the flagged-workgroup list and two
// digit histograms.
// Plain rows over at most kSampleMaxS workgroups take their threshold from a
// sample of the row (split_kernel); the regions are laid out in units of 64
// slots, kCapF / 64 of them.
constexpr int kSampleMaxS = 64;
constexpr uint32_t kSampleMaxK = 1024;
constexpr uint32_t kSpreadC = 96; // see the mode word (split_kernel)
constexpr uint32_t kUnits = (uint32_t)kCapF / 64u;
static_assert(kUnits * 64u == (uint32_t)kCapF && kUnits <= 128u, "whole units, one byte each");
constexpr int kPoolWords = 38912;                      // 152 KiB
constexpr int kStageOff = 1024 + 2 * HistBuf<12>::NB;  // list, then two histograms
constexpr uint32_t kStageWords = (uint32_t)(kPoolWords - kStageOff); // 29,696 keys

template <int T, int E, int MODE, bool WHOLE>
__global__ __launch_bounds__(T) void split_kernel(KParams p)
{
    constexpr int MAXW = 12;
    constexpr int NB = HistBuf<MAXW>::NB;
    constexpr int NW = T / 64;
    static_assert(kStageOff == 1024 + 2 * NB && kMaxS <= 1024, "pool layout");
    // Instances whose recovery stages chunks in LDS: the exchange instances of
    // plain rows with four scores per thread and of the block stage with one
    // block per thread. (Candidate slots do not carry their index; the
    // instances with more elements per thread are at the register limit
    // already, and the staged select would make them spill.)
    constexpr bool STAGED = !WHOLE && ((MODE == MODE_PLAIN && E == 4) || (MODE == MODE_BLOCKS && E == 1));
    // Instances that may take the row's threshold from a sample: plain rows
    // of four scores per thread (64 sampled scores per chunk of 4096).
    constexpr bool SAMPLED = !WHOLE && MODE == MODE_PLAIN && E == 4;
    // three rotating digit histograms (block_regs_select); the third also
    // holds the histograms of the local bound and of the exact fallback. In
    // the rows' exchange instances the rest of the pool is the recovery's
    // staging area.
    __shared__ __attribute__((aligned(16))) uint32_t pool[STAGED ? kPoolWords : 3 * NB];
    uint32_t *const hbuf = pool;
    uint32_t *const hist = hbuf + 2 * NB;
    __shared__ uint32_t pubcnt[kMaxS];
    __shared__ uint32_t wtop;
    __shared__ uint64_t mred[4 * NW];
    __shared__ uint32_t tmp[NW];
    __shared__ uint32_t res[4];
    __shared__ uint32_t bc[4];
    __shared__ uint32_t ectr;
    // sampled rows: per-chunk sample counts [0, 64), the region layout
    // [64, 128) (first unit | units << 8), the unit table [128, 256)
    __shared__ uint32_t lay[SAMPLED ? 256 : 1];
    __shared__ uint32_t cmax; // last workgroup: most slots a workgroup published
    __shared__ uint32_t sjn;  // sampled rows: the sample rank of the threshold
    // last workgroup of rows of four scores per thread: the select's key
    // check (a word per wave) and the tie break's counts
    __shared__ uint32_t kwd[SAMPLED ? NW : 1];
    __shared__ uint32_t tcnt[SAMPLED ? 128 : 1];

    const int row = p.row0 + (int)blockIdx.y;
    const uint32_t S = gridDim.x;
    const uint32_t g = blockIdx.x;
    const int32_t len = row_len(p, row);
    const uint32_t k = (uint32_t)p.k;
    int32_t *out = p.out + (int64_t)row * p.k;
    const int ibits = index_bits(MODE == MODE_BLOCKS ? p.vlen : (int64_t)p.n_max);

    block_zero<T>(hbuf, 3 * NB);
    if (threadIdx.x == 0)
        wtop = 0u;
    // Rows that may sample keep a mode word in their workspace record, left
    // by the previous call on it: 0, each workgroup bounds its candidates by
    // its own scores (cheapest when the row's best scores are spread out);
    // 1, by a threshold taken from a sample of the whole row (exact without
    // a second pass when they cluster in a few chunks). A call in mode 0
    // that needed the second pass sets 1; a call in mode 1 whose workgroups
    // all published few candidates sets 0. Both modes give the same result.
    // The sample (issued with the mode word and before the chunk, so that
    // the loads are in flight together): 64 scores of every chunk, in four
    // runs of 16 that start 1024 apart at offsets varying by chunk (the
    // first run of chunk 0 opens the row); one 16-byte load per thread,
    // threads 16 c .. 16 c + 15 on chunk c.
    const bool may_sample = SAMPLED && S > 1u && S <= (uint32_t)kSampleMaxS && k <= kSampleMaxK;
    uint32_t modew = 0u;
    u4 smp = {0u, 0u, 0u, 0u};
    uint32_t spos = 0u;
    bool shas = false;
    uint32_t key[E], nid[E];
    if constexpr (SAMPLED) {
        // The chunk's loads, then the sample's, then the mode word's, none
        // behind a branch (an empty range, a zero word when not sampling):
        // the keys then wait for the chunk alone, and nothing waits for the
        // mode word before the first barrier.
        const float *x = p.scores + (int64_t)row * p.row_stride;
        const int64_t base = (int64_t)g * T * E;
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(x, base, len);
        u4 f[E / 4];
#pragma unroll
        for (int v = 0; v < E / 4; ++v)
            f[v] = load16(rs, (uint32_t)(v * T + threadIdx.x) * 16u);
        {
            const uint32_t c = threadIdx.x >> 4, q = (threadIdx.x >> 2) & 3u;
            shas = may_sample && c < S;
            spos = c * (uint32_t)(T * E) + q * (uint32_t)(T * E / 4) +
                   (((c * 5u + q * 3u) & 63u) << 4) + ((threadIdx.x & 3u) << 2);
            smp = load16(row_rsrc(x, 0, shas ? len : 0), spos * 4u);
            const uint32_t *mw = may_sample ? p.ws + (int64_t)blockIdx.y * kWsRowWords + kWsMode
                                            : &g_zero_word;
            modew = __hip_atomic_load(mw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int v = 0; v < E / 4; ++v) {
            const int64_t v0 = base + ((int64_t)v * T + threadIdx.x) * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                key[4 * v + j] = (v0 + j < len) ? score_key(f[v][j]) : 0u;
                nid[4 * v + j] = ~(uint32_t)(v0 + j);
            }
        }
    } else {
        Loader<T, E, MODE>::load(p, row, len, (int64_t)g * T * E, key, nid);
    }
    uint32_t nvalid = 0, tmax = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        nvalid += key[j] != 0u ? 1u : 0u;
        tmax = key[j] > tmax ? key[j] : tmax;
    }

    if (WHOLE || S == 1) {
        // ---- the whole row is in this workgroup: exact select over registers
        uint32_t V;
        (void)block_excl_prefix<T>(nvalid, tmp, V);
        const uint32_t m = V < k ? V : k;
        SelState st = sel_start(V, m);
        block_regs_select<T, MAXW>(key, nid, st, 0u, hbuf, tmp, res, ibits);
        const uint64_t F = sel_floor(st);
        const uint32_t fk = (uint32_t)(F >> 32), fn = (uint32_t)F;
        uint32_t nsel = 0;
#pragma unroll
        for (int j = 0; j < E; ++j)
            nsel += at_or_above(key[j], nid[j], fk, fn) ? 1u : 0u;
        uint32_t tot;
        uint32_t slot = block_excl_prefix<T>(nsel, tmp, tot);
#pragma unroll
        for (int j = 0; j < E; ++j) {
            if (at_or_above(key[j], nid[j], fk, fn)) {
                if (slot < m)
                    out[slot] = (int32_t)~nid[j];
                ++slot;
            }
        }
        for (uint32_t i = m + threadIdx.x; i < k; i += T)
            out[i] = -1;
        return;
    }

    // ---- S > 1: publish a local candidate set that provably covers this
    // workgroup's part of the row's top-m, then take a ticket.
    uint32_t *ws = p.ws + (int64_t)blockIdx.y * kWsRowWords;
    // Share r of the row's top-k this workgroup must cover: its expected
    // share (k times its fraction of the row's valid elements) plus four
    // standard deviations of a binomial share and a margin of 16. A workgroup
    // holding more is caught by the check in the last workgroup. Every
    // workgroup of the row sizes the regions alike (R slots): four times the
    // largest share, capped so that the row's regions fit the workspace.
    // Computed by the first wave alone and handed to the others through LDS
    // at the barriers below: uniform arithmetic run by all sixteen waves
    // would cost sixteen times over.
    if (threadIdx.x < 64) {
        constexpr uint32_t C = (uint32_t)T * E;
        const uint32_t vl = (uint32_t)virtual_len(p, MODE, len);
        const float inv = vl > 0u ? __builtin_amdgcn_rcpf((float)vl) : 0.0f;
        auto share = [&](uint32_t mine) {
            const float mu = __builtin_ceilf((float)k * (float)mine * inv);
            return mu + 4.0f * __builtin_amdgcn_sqrtf(mu) + 16.0f;
        };
        const uint32_t done = g * C;
        uint32_t mine = vl > done ? vl - done : 0u; // elements of this workgroup (plain, blocks)
        mine = MODE == MODE_CAND ? C : (mine > C ? C : mine);
        const uint32_t cap = (uint32_t)kCapF / S;
        const float rmax = 4.0f * share(MODE == MODE_CAND || vl > C ? C : vl);
        const uint32_t R0 = rmax >= (float)cap ? cap : (uint32_t)rmax;
        const float want = share(mine);
        if (threadIdx.x == 0) {
            bc[2] = want >= (float)R0 ? R0 : (uint32_t)want;
            bc[3] = R0;
            if (may_sample) {
                // Sampled threshold: the sample's j-th best score, j chosen
                // so that the row's m-th best lies above it with overwhelming
                // odds (each sampled score stands for 64: j covers m / 64
                // plus 4.5 standard deviations and 4); about 64 j scores are
                // then published in all.
                const uint32_t m0 = (uint32_t)len < k ? (uint32_t)len : k;
                const float mu = (float)m0 * (1.0f / 64.0f);
                sjn = (uint32_t)__builtin_ceilf(mu + 4.5f * __builtin_amdgcn_sqrtf(mu) + 4.0f);
            }
        }
    }

    // Mode 0: a cheap local bound from the per-thread maxima (the 12-bit
    // bin where r of them are reached from the top has at least r elements
    // at or above it). Mode 1: the sample's 12-bit histogram (lanes sharing
    // lane 0's bin add once, through lane 0: rows where most scores are -inf
    // or one repeated value would otherwise serialise on one LDS word).
    __syncthreads();
    const bool sampled =
        may_sample && (p.force_sample == 2u || (p.force_sample == 0u && uni(modew) != 0u));
    uint32_t skey[4] = {0u, 0u, 0u, 0u};
    if (sampled) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            skey[j] = shas && spos + (uint32_t)j < (uint32_t)len ? score_key(smp[j]) : 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t b = skey[j] >> 20;
            const uint32_t lead = uni(b);
            const uint64_t same = __ballot(skey[j] != 0u && b == lead);
            if (skey[j] != 0u && b != lead)
                atomicAdd(&hist[b], 1u);
            if ((threadIdx.x & 63u) == 0u && same != 0ull)
                atomicAdd(&hist[lead], (uint32_t)__popcll(same));
        }
    } else if (tmax != 0u) {
        atomicAdd(&hist[tmax >> 20], 1u);
    }
    {
        // the workgroup's largest key bounds its candidates from above
        const uint32_t wm = wave_max_u32(tmax);
        if ((threadIdx.x & 63) == 0)
            atomicMax(&wtop, wm);
    }
    __syncthreads();
    uint32_t r, R, roff;
    bool found;
    SelState st = sel_start(nvalid, 0u);
    st.s = 52;
    if (sampled) {
        // every workgroup reads the same sample, so every workgroup finds the
        // same threshold bin and the same region layout, with no exchange
        const uint32_t jn = uni(sjn);
        const BinHit th = block_find_bin<T>(hist, NB, jn, tmp, res);
        // threshold: the 22-bit key prefix of the sample's j-th best (a
        // 12-bit bin alone can hold twice the wanted count above its floor)
        uint32_t bin = 0u;
        if (th.total >= jn) {
            uint32_t *const h2 = hbuf; // still zero
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if ((skey[j] >> 20) == th.bin)
                    atomicAdd(&h2[(skey[j] >> 10) & 1023u], 1u);
            __syncthreads();
            const BinHit t2 = block_find_bin<T>(h2, 1024, jn - th.above, tmp, res);
            bin = (th.bin << 10) | t2.bin;
            h2[threadIdx.x] = 0u; // (ordered before the next use by the barriers below)
        }
        uint32_t e = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            e += skey[j] != 0u && (skey[j] >> 10) >= bin ? 1u : 0u;
        // sum over the 16 lanes of a DPP row: one chunk's sample
        e += dpp<0x111, 0xf>(e, 0u);
        e += dpp<0x112, 0xf>(e, 0u);
        e += dpp<0x114, 0xf>(e, 0u);
        e += dpp<0x118, 0xf>(e, 0u);
        if ((threadIdx.x & 15u) == 15u && shas)
            lay[threadIdx.x >> 4] = e;
        __syncthreads();
        if (threadIdx.x < 64) {
            // Regions in units of 64 slots: one per chunk, and the spare
            // units shared in proportion to the chunks' sampled counts above
            // the bin (floors, so the units never exceed kUnits).
            const uint32_t l = threadIdx.x;
            const uint32_t ec = l < S ? lay[l] : 0u;
            const uint32_t et = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_prefix(ec), 63);
            const uint32_t spare = kUnits - S;
            const uint32_t un = l < S ? 1u + (et != 0u ? spare * ec / et : spare / S) : 0u;
            const uint32_t ou = wave_incl_prefix(un) - un;
            if (l < S)
                lay[64 + l] = ou | (un << 8);
        }
        __syncthreads();
        const uint32_t lw = uni(lay[64 + g]);
        R = 64u * (lw >> 8);
        roff = 64u * (lw & 255u);
        r = R;
        found = true;
        st.s = 42;
        st.P = bin;
    } else {
        r = uni(bc[2]);
        R = uni(bc[3]);
        roff = g * R;
        const BinHit th = block_find_bin<T>(hist, NB, r, tmp, res);
        found = th.total >= r;
        st.P = found ? th.bin : 0u;
    }
    uint32_t npub = 0;
    const uint32_t psh = (uint32_t)(st.s - 32); // the bound's digits cover key bits psh..31
#pragma unroll
    for (int j = 0; j < E; ++j)
        npub += (key[j] != 0u && (key[j] >> psh) >= (uint32_t)st.P) ? 1u : 0u;
    uint32_t tot;
    // (no closing barrier: tmp is next written after the ticket's barrier,
    // or after the one that opens the narrowing below)
    uint32_t ex = block_excl_prefix<T, false>(nvalid | (npub << 16), tmp, tot);
    const uint32_t nvalid_g = tot & 0xffffu;
    uint32_t c = tot >> 16;
    if (!found || c > R) {
        // Too few maxima, or too many elements share the bound's bin: narrow
        // down with exact local digits until the published set fits.
        // The select starts below the key bits that the bound and the
        // workgroup's largest key share: the c elements at or above the
        // bound (more than R >= need of them) lie in that range, and those
        // below it that share its prefix fall in bins under the cut.
        __syncthreads();
        const uint32_t need = min(min(r, R), nvalid_g);
        st = sel_start_range(found ? sel_floor(st) : 0ull,
                             ((uint64_t)uni(wtop) << 32) | 0xffffffffull, found ? c : nvalid_g,
                             need);
        block_regs_select<T, MAXW, E, true>(key, nid, st, R, hbuf, tmp, res, ibits);
        if (st.s == 32 && st.cnt != st.need && st.above + st.cnt > R) {
            // More than R elements tie on one key K (attention sinks, a
            // constant stretch). Ordering them by index here would take a
            // pass per index digit; publish only the keys above K instead
            // (fewer than r of them). The bound then says every unpublished
            // element has a key below K + 1, and if the ties matter the last
            // workgroup re-reads this chunk.
            st.P += 1u;
        }
        npub = 0;
#pragma unroll
        for (int j = 0; j < E; ++j)
            npub += (key[j] != 0u && pfx(comp(key[j], nid[j]), st.s) >= st.P) ? 1u : 0u;
        ex = block_excl_prefix<T>(npub << 16, tmp, tot);
        c = tot >> 16;
    }
    // publish: (key, ~index) composites in slots [0, c) of the region; the
    // meta record says how many slots are valid
    uint64_t *region = reinterpret_cast<uint64_t *>(ws + kWsRegion) + roff;
    uint32_t slot = ex >> 16;
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const uint64_t cc = comp(key[j], nid[j]);
        if (key[j] != 0u && pfx(cc, st.s) >= st.P) {
            if (slot < R)
                put64(region + slot, cc);
            ++slot;
        }
    }
    if (threadIdx.x == 0) {
        // every unpublished element of this workgroup lies below `bound`
        // meta word 0: valid count (bits 0-15), published count (16-29),
        // truncated flag (30), largest key (32-63); word 1: the bound
        const uint32_t cpub = c < R ? c : R;
        uint64_t *meta = reinterpret_cast<uint64_t *>(ws + kWsMeta) + 2 * (int64_t)g;
        put64(meta, ((uint64_t)wtop << 32) | ((nvalid_g > cpub ? 1u : 0u) << 30) | (cpub << 16) |
                        nvalid_g);
        put64(meta + 1, sel_floor(st));
    }

    // ---- ticket: the last workgroup of the row finishes it
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t t = __hip_atomic_fetch_add(ws + kWsTicket, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        bc[0] = (t == S - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (bc[0] == 0u)
        return;

    // ---- last workgroup: gather, select, verify
    // Every published slot is loaded into registers in one round trip (slot
    // i = g * R + j of the region is valid when j < count_g); the metas come
    // in the same round trip.
    constexpr int G = (kCapF + T - 1) / T;
    const uint32_t n = sampled ? (uint32_t)kCapF : S * R;
    const uint64_t *rsrc = reinterpret_cast<const uint64_t *>(ws + kWsRegion);
    const uint64_t *meta = reinterpret_cast<const uint64_t *>(ws + kWsMeta);
    uint64_t v[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const uint32_t i = threadIdx.x + (uint32_t)j * T;
        v[j] = i < n ? get64(rsrc + i) : 0ull;
    }
    // metas: thread i < S holds workgroup i's; the waves holding any reduce
    // them (valid total, published total, lowest bound of a workgroup that
    // published, largest key, highest bound of a truncated workgroup)
    static_assert(kMaxS <= T, "one meta record per thread");
    uint32_t gvalid = 0; // thread g < S: valid elements of workgroup g
    uint64_t gtrunc = 0; // thread g < S: its bound if it left elements out, else 0
    {
        uint32_t vs = 0, cs = 0, top = 0;
        uint64_t lob = ~0ull, trb = 0ull;
        if (threadIdx.x < S) {
            const uint64_t m0 = get64(meta + 2 * threadIdx.x);
            const uint64_t b0 = get64(meta + 2 * threadIdx.x + 1);
            const uint32_t cp = (uint32_t)(m0 >> 16) & 0x3fffu;
            vs = (uint32_t)m0 & 0xffffu;
            cs = cp;
            top = (uint32_t)(m0 >> 32);
            lob = cp != 0u ? b0 : ~0ull;
            trb = ((m0 >> 30) & 1u) ? b0 : 0ull;
            pubcnt[threadIdx.x] = cp;
            gvalid = vs;
            gtrunc = trb;
        }
        if (sampled && threadIdx.x < 64) {
            const uint32_t cm = wave_max_u32(threadIdx.x < S ? pubcnt[threadIdx.x] : 0u);
            if (threadIdx.x == 0)
                cmax = cm;
        }
        if (sampled && threadIdx.x < 64) {
            // Unit table (first wave, units 2 l and 2 l + 1 on lane l): the
            // chunk a unit belongs to (each chunk's first unit marked, then a
            // running maximum) and how many of its 64 slots were published,
            // as valid | chunk << 8.
            const uint32_t l = threadIdx.x;
            uint32_t *const ut = lay + 128;
            ut[2 * l] = 0u;
            ut[2 * l + 1] = 0u;
            wave_sync();
            if (l < S)
                ut[lay[64 + l] & 255u] = l + 1u;
            wave_sync();
            const uint32_t a0 = ut[2 * l], a1 = ut[2 * l + 1];
            uint32_t inc = a0 > a1 ? a0 : a1;
            inc = max(inc, dpp<0x111, 0xf>(inc, 0u));
            inc = max(inc, dpp<0x112, 0xf>(inc, 0u));
            inc = max(inc, dpp<0x114, 0xf>(inc, 0u));
            inc = max(inc, dpp<0x118, 0xf>(inc, 0u));
            inc = max(inc, dpp<0x142, 0xa>(inc, 0u));
            inc = max(inc, dpp<0x143, 0xc>(inc, 0u));
            const uint32_t prev = dpp<0x138, 0xf>(inc, 0u); // wave_shr:1
            const uint32_t c0 = (prev > a0 ? prev : a0) - 1u, c1 = inc - 1u;
            auto valid_in = [&](uint32_t b, uint32_t cc) {
                const int d = (int)pubcnt[cc] - 64 * ((int)b - (int)(lay[64 + cc] & 255u));
                return (uint32_t)(d < 0 ? 0 : (d > 64 ? 64 : d)) | (cc << 8);
            };
            const uint32_t u0 = valid_in(2 * l, c0), u1 = valid_in(2 * l + 1, c1);
            wave_sync();
            ut[2 * l] = u0;
            ut[2 * l + 1] = u1;
        }
        const uint32_t w = threadIdx.x >> 6;
        if (uni(w * 64u) < S) {
            vs = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_prefix(vs), 63);
            cs = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_prefix(cs), 63);
            top = wave_max_u32(top);
            lob = wave_min_u64(lob);
            trb = wave_max_u64(trb);
            if ((threadIdx.x & 63) == 0) {
                mred[w] = ((uint64_t)cs << 32) | vs;
                mred[NW + w] = top;
                mred[2 * NW + w] = lob;
                mred[3 * NW + w] = trb;
            }
        }
    }
    block_zero<T>(hbuf, 2 * NB);
    if (threadIdx.x == 0) {
        ectr = 0u;
    }
    __syncthreads();
    uint32_t V = 0, ncand = 0, top = 0;
    uint64_t lo = ~0ull, maxb = 0ull;
    for (uint32_t w = 0; w * 64u < S; ++w) {
        const uint64_t a = mred[w];
        V += (uint32_t)a;
        ncand += (uint32_t)(a >> 32);
        top = (uint32_t)mred[NW + w] > top ? (uint32_t)mred[NW + w] : top;
        lo = mred[2 * NW + w] < lo ? mred[2 * NW + w] : lo;
        maxb = mred[3 * NW + w] > maxb ? mred[3 * NW + w] : maxb;
    }
    const uint64_t hi = ((uint64_t)top << 32) | 0xffffffffull;
    uint32_t ckey[G], cnid[G];
    if (sampled) {
        // slot i = threadIdx.x + j * T lies in unit (wave + 16 j): valid when
        // its lane is below the unit's published count
        const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const uint32_t b = w + (uint32_t)j * (T / 64);
            const uint32_t u = b < kUnits ? uni(lay[128 + b]) : 0u;
            ckey[j] = lane < (u & 255u) ? (uint32_t)(v[j] >> 32) : 0u;
            cnid[j] = (uint32_t)v[j];
        }
    } else {
        // (group, slot) of i = threadIdx.x + j * T, advanced incrementally;
        // counts are read four at a time so their LDS reads overlap
        uint32_t g0 = threadIdx.x / R, s0 = threadIdx.x - g0 * R;
        const uint32_t dq = (uint32_t)T / R, dr = (uint32_t)T - dq * R;
        static_assert(G % 4 == 0, "slots are checked in fours");
#pragma unroll
        for (int j0 = 0; j0 < G; j0 += 4) {
            uint32_t sl[4], pc[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                sl[q] = s0;
                pc[q] = pubcnt[g0 < S ? g0 : 0u];
                g0 += dq;
                s0 += dr;
                const bool carry = s0 >= R;
                s0 = carry ? s0 - R : s0;
                g0 = carry ? g0 + 1u : g0;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = j0 + q;
                const uint32_t i = threadIdx.x + (uint32_t)j * T;
                const bool valid = i < n && sl[q] < pc[q];
                ckey[j] = valid ? (uint32_t)(v[j] >> 32) : 0u;
                cnid[j] = (uint32_t)v[j];
            }
        }
    }
    const uint32_t Vt = V;
    const uint32_t m = Vt < k ? Vt : k;

    bool ok = p.force_fallback == 0u;
    SelState fs = sel_start_range(lo, hi, ncand, m);
    if (ok && m > 0u) {
        if constexpr (SAMPLED) {
            // Here the slots hold the candidates in index order (regions
            // follow the chunks; a workgroup publishes in position order),
            // so ties on the last key are broken by slot order. The ties it
            // drops lie below the selection; every bound a workgroup
            // publishes has zero index bits, so the check against the lower
            // edge (K, 0) decides as against the exact one, and the second
            // pass still holds m candidates at or above it.
            block_regs_select<T, MAXW, G, false, true>(ckey, cnid, fs, 0u, hbuf, tmp, res, ibits,
                                                       kwd);
            if (fs.s <= 32 && fs.cnt > fs.need)
                tie_floor_slots<T, G>(ckey, cnid, fs, tcnt);
        } else {
            block_regs_select<T, MAXW>(ckey, cnid, fs, 0u, hbuf, tmp, res, ibits);
        }
        // exact only if no truncated workgroup can hide an element at or
        // above the selection's lower edge
        ok = fs.cnt == fs.need && maxb <= sel_floor(fs);
    }
    if (ok) {
        const uint64_t F = sel_floor(fs);
        const uint32_t fk = m != 0u ? (uint32_t)(F >> 32) : 0xffffffffu;
        const uint32_t fn = m != 0u ? (uint32_t)F : 0xffffffffu;
        uint32_t ns = 0;
#pragma unroll
        for (int j = 0; j < G; ++j)
            ns += at_or_above(ckey[j], cnid[j], fk, fn) ? 1u : 0u;
        // output order is free: each wave takes its slots with one LDS atomic
        // on a counter zeroed before the select, no block-wide scan
        const uint32_t inc = wave_incl_prefix(ns);
        const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
        uint32_t base = 0;
        if ((threadIdx.x & 63) == 0 && wtot != 0u)
            base = atomicAdd(&ectr, wtot);
        uint32_t q = (uint32_t)__builtin_amdgcn_readlane((int)base, 0) + inc - ns;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            if (at_or_above(ckey[j], cnid[j], fk, fn)) {
                if (q < m)
                    out[q] = (int32_t)~cnid[j];
                ++q;
            }
        }
    } else if (p.force_fallback == 0u && fs.cnt == fs.need) {
        // The check failed: some workgroups left out elements at or above the
        // selection's floor F0 (their winners cluster). Every other element
        // left out lies below F0, and at least m published ones reach it, so
        // the top-m of the row is the top-m of: the published candidates of
        // the other workgroups, plus every element of the flagged ones.
        const uint64_t F0 = sel_floor(fs);
        if (threadIdx.x < S)
            pubcnt[threadIdx.x] = gtrunc > F0 ? 1u : 0u; // (read before the select's barriers)
        if (threadIdx.x == 0)
            bc[1] = 0u;
        __syncthreads();
        uint32_t u = threadIdx.x < S && gtrunc > F0 ? gvalid : 0u;
        if constexpr (!STAGED) {
            // (the division costs ~1 us per recovery, but the incremental form
            // below needs registers these instances have not)
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const uint32_t i = threadIdx.x + (uint32_t)j * T;
                if (i < n && pubcnt[i / R] != 0u)
                    ckey[j] = 0u;
                u += ckey[j] != 0u ? 1u : 0u;
            }
        } else if (sampled) {
            // group of slot i = threadIdx.x + j * T: the unit table's
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const uint32_t b = (threadIdx.x >> 6) + (uint32_t)j * (T / 64);
                if (b < kUnits && pubcnt[uni(lay[128 + b]) >> 8] != 0u)
                    ckey[j] = 0u;
                u += ckey[j] != 0u ? 1u : 0u;
            }
        } else {
            // group of slot i = threadIdx.x + j * T, advanced as in the gather
            uint32_t g0 = threadIdx.x / R, s0 = threadIdx.x - g0 * R;
            const uint32_t dq = (uint32_t)T / R, dr = (uint32_t)T - dq * R;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const uint32_t i = threadIdx.x + (uint32_t)j * T;
                if (i < n && pubcnt[g0 < S ? g0 : 0u] != 0u)
                    ckey[j] = 0u;
                u += ckey[j] != 0u ? 1u : 0u;
                g0 += dq;
                s0 += dr;
                const bool carry = s0 >= R;
                s0 = carry ? s0 - R : s0;
                g0 = carry ? g0 + 1u : g0;
            }
        }
        const uint32_t ut = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_prefix(u), 63);
        if ((threadIdx.x & 63) == 0 && ut != 0u)
            atomicAdd(&bc[1], ut);
        // the flagged workgroups as a list (in the first histogram buffer,
        // which the re-read select does not use), built by the first wave
        uint32_t *const list = hbuf;
        if (threadIdx.x < 64) {
            uint32_t nf = 0;
            for (uint32_t g0 = 0; g0 < S; g0 += 64) {
                const uint32_t g = g0 + threadIdx.x;
                const bool f = g < S && pubcnt[g] != 0u;
                const uint64_t mk = __ballot(f);
                if (f)
                    list[nf + lane_rank(mk)] = g;
                nf += (uint32_t)__popcll(mk);
            }
            if (threadIdx.x == 0)
                bc[2] = nf;
        }
        __syncthreads();
        const uint32_t nl = uni(bc[2]);
        bool staged = false;
        if constexpr (STAGED) {
            // the flagged chunks fit LDS: load them once, select there
            if (nl * (uint32_t)(T * E) <= kStageWords)
                staged = staged_part_select<T, E, MODE, MAXW>(
                    p, row, len, list, nl, F0, hi, uni(bc[1]), m, ckey, cnid, out,
                    pool + kStageOff, pool + 1024, pool + 1024 + NB,
                    reinterpret_cast<uint32_t *>(mred), tmp, res, ibits);
        }
        if (!staged)
            block_part_select<T, E, MODE, MAXW>(p, row, len, list, nl, F0, hi, uni(bc[1]), m,
                                                ckey, cnid, out, hist, tmp, res, &ectr);
    } else {
        __syncthreads(); // every wave is done reading the select's histograms
        block_row_select<T, E, MODE, MAXW>(p, row, len, Vt, m, out, hist, tmp, res, &bc[1]);
    }
    for (uint32_t i = m + threadIdx.x; i < k; i += T)
        out[i] = -1;
    if (threadIdx.x == 0) {
        if (may_sample) {
            // the next call's mode: sample after a second pass; stop sampling
            // once no workgroup holds more than kSpreadC candidates (a spread
            // row, which the cheaper mode serves in one pass)
            const uint32_t next = sampled ? (cmax > kSpreadC ? 1u : 0u) : (ok ? 0u : 1u);
            __hip_atomic_store(ws + kWsMode, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __hip_atomic_store(ws + kWsTicket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ------------------------------------------------------------------ stream kernel

// Float threshold for the strict test "score_key(x) > T" (T a key a compaction
// produced, T >= 1): x >= result holds exactly when score_key(x) > T. It is
// the score whose key is T + 1 (any key in the NaN range maps to -inf, so
// every non-NaN score passes; keys above +inf's map to a NaN, so none does);
// -0.0 needs no key of its own because both zeros compare equal as floats.
__device__ __forceinline__ float key_floor_float(uint32_t T)
{
    const uint32_t t1 = T + 1u;
    const uint32_t bits = t1 <= 0x007fffffu ? 0xff800000u
                          : (t1 >= 0x80000000u ? (t1 ^ 0x80000000u) : ~t1);
    return __uint_as_float(bits);
}

// Floor composite by radix select over a streaming buffer (the rare path of
// its compactions and of its final selection). The entries >= the
// returned floor number `want` (limit 0) or lie in [want, limit]. With
// `armed` every entry's key is >= thr and <= kbound; otherwise the buffer may
// hold empty slots and the range is measured first. Clobbers hist.
struct FloorPick {
    uint64_t F;
    uint32_t kmax; // bound on the keys of the entries >= F
    bool any;      // false: keep nothing
};

template <int MAXW>
__device__ __forceinline__ FloorPick stream_select_floor(const uint32_t *lkey, const uint32_t *lnid,
                                                      uint32_t *hist, uint32_t n_buf, bool armed,
                                                      uint32_t thr, uint32_t kbound,
                                                      uint32_t want, uint32_t limit)
{
    const int lane = threadIdx.x & 63;
    uint64_t lo, hi;
    uint32_t cnt = n_buf;
    if (armed) {
        lo = (uint64_t)thr << 32;
        hi = ((uint64_t)kbound << 32) | 0xffffffffull;
    } else {
        uint32_t c = 0;
        uint64_t mn = ~0ull, mx = 0ull;
        for (uint32_t i0 = 0; i0 < n_buf; i0 += 512) {
            uint32_t kk[8], nn[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t i = i0 + q * 64 + lane;
                kk[q] = i < n_buf ? lkey[i] : 0u;
                nn[q] = i < n_buf ? lnid[i] : 0u;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint64_t cc = comp(kk[q], nn[q]);
                if (kk[q] != 0u) {
                    ++c;
                    mn = cc < mn ? cc : mn;
                    mx = cc > mx ? cc : mx;
                }
            }
        }
        cnt = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_prefix(c), 63);
        lo = wave_min_u64(mn);
        hi = wave_max_u64(mx);
    }
    if (want > cnt)
        want = cnt;
    SelState st = sel_start_range(lo, hi, cnt, want);
    wave_lds_select<MAXW>(lkey, lnid, n_buf, st, hist, limit);
    FloorPick r;
    r.F = sel_floor(st);
    r.kmax = (uint32_t)(hi >> 32);
    r.any = want != 0u;
    return r;
}

// Per-mode shape of a streaming sweep: 16-byte loads per lane (LPS) and
// elements per lane (EPL). Plain rows: four consecutive scores. Candidates
// (blocks of eight): half a block per lane, a lane pair per block. Block
// stage (blocks of eight): two blocks per lane, each scored by its best key.
template <int MODE>
struct StreamShape {
    static constexpr int LPS = MODE == MODE_BLOCKS ? 4 : 1;
    static constexpr int EPL = MODE == MODE_BLOCKS ? 2 : 4;
};

// One wave per row; the row (or its candidate blocks) is read once with PD
// sweeps in flight. Until the LDS buffer is first compacted every element is
// kept (absent ones as empty slots). After that an element enters only if its
// key passes the admission threshold thr, a key that at least k kept elements
// reach. Plain rows are read from their end backwards: the recent positions
// of a causal row tend to score highest, so the threshold is high from the
// first sweeps on, and a row that rises toward the present admits little
// after them (read forwards, nearly every score of such a row would enter).
// Read backwards, a later element whose key equals thr has a lower index than
// the kept ones and outranks them, so the test admits key >= thr; candidate
// blocks come in list order, where the same holds. The cost falls on rows
// whose best scores come first or that tie heavily at the threshold: there
// more elements enter, and the selection stays exact. Blocks are read in
// index order (backwards measured 3 % slower on i.i.d. rows), so a later
// block whose key equals thr can never displace a kept one and their test is
// strict (key > thr). Plain rows and candidates test the float scores
// themselves (one compare per score, key_floor_float); blocks test their
// integer key. After every sweep a buffer above CAPS = BUF - SWEEP is
// compacted to between k and keep_limit (halfway between k and CAPS) entries,
// thr becoming the smallest key kept. One sweep of headroom above CAPS means
// a sweep always fits. Once armed, the wave keeps a 256-bin histogram of the
// buffer's keys, updated on every append, so a compaction reads the new thr
// off it (the lower edge of the bin holding the k-th largest) and makes one
// pass over the buffer; the first compaction takes thr from a radix select
// on the buffer's first 512 entries, checked by one counting pass. Radix
// select over the whole buffer is the fallback for both. The final exact
// selection ranks the k-th largest's bin alone: one entry per lane if it has
// at most 64, else by radix select from that bin's key prefix.
template <int MODE, int BUF, int PD, int MAXW, bool LONG>
__global__ __launch_bounds__(64) void stream_kernel(KParams p)
{
    constexpr int LPS = StreamShape<MODE>::LPS;
    constexpr int EPL = StreamShape<MODE>::EPL;
    constexpr int SWEEP = 64 * EPL;         // elements per sweep
    constexpr int CAPS = BUF - SWEEP;       // compact above this (checked every sweep)
    constexpr bool REV = MODE == MODE_PLAIN;    // sweeps visited from the row's end
    constexpr bool STRICT = MODE == MODE_BLOCKS; // admission test key > thr (else >=)
    static_assert(CAPS >= SWEEP, "the buffer must hold two sweeps");
    __shared__ __attribute__((aligned(16))) uint32_t lkey[BUF];
    __shared__ __attribute__((aligned(16))) uint32_t lnid[BUF];
    __shared__ __attribute__((aligned(16))) uint32_t hist[(1 << MAXW) < 256 ? 256 : (1 << MAXW)];

    const int lane = threadIdx.x;
    const int row = p.row0 + (int)blockIdx.x;
    const int32_t len = row_len(p, row);
    const uint32_t k = (uint32_t)p.k;
    const uint32_t keep_limit = (k + (uint32_t)CAPS) / 2u; // the host keeps k < CAPS
    const float *x = p.scores + (int64_t)row * p.row_stride;
    int32_t *out = p.out + (int64_t)row * p.k;
    // elements of the virtual row: positions, blocks, or candidate slots
    const int32_t nel = MODE == MODE_PLAIN ? len
                        : (MODE == MODE_BLOCKS ? (len + 7) / 8 : p.n_cand * 8);

    uint32_t n_buf = 0;   // slots used (wave-uniform)
    uint32_t thr = 0;     // admission threshold key once armed
    float tf = 0.0f;      // the same threshold as a float (plain rows, candidates)
    uint32_t kmax = 0;    // per lane: bound on the keys this lane appended
    bool armed = false;

    // Histogram of the buffer's keys, kept while armed: every entry's key is
    // >= hb, and bin min((key - hb) >> hs, 255) counts it. hb is aligned to
    // 1 << hs, so each bin below the top one is the set of keys with one
    // prefix. With it a compaction needs no pass to find its threshold.
    constexpr uint32_t kHB = 256u;
    uint32_t hb = 0, hs = 0;
    auto hbin = [&](uint32_t kk) {
        const uint32_t b = (kk - hb) >> hs;
        return b < kHB - 1u ? b : kHB - 1u;
    };

    auto select_floor = [&](uint32_t want, uint32_t limit, uint64_t &F) {
        const FloorPick r = stream_select_floor<MAXW>(lkey, lnid, hist, n_buf, armed, thr,
                                                      armed ? wave_max_u32(kmax) : 0u, want, limit);
        F = r.F;
        kmax = uni(r.kmax);
        return r.any;
    };

    // Without a histogram (the first compaction): a key T picked by radix
    // select on the first 512 entries, at the rank that would put the full
    // buffer's count between k and keep_limit, then one counting pass. If
    // the count lands there, F = T << 32 (every entry with key >= T kept);
    // else false, and the caller selects over the whole buffer.
    auto sample_floor = [&](uint64_t &F) {
        constexpr uint32_t kS = 512;
        if (n_buf < 2u * kS)
            return false;
        const uint32_t r = (uint32_t)((uint64_t)kS * ((k + keep_limit) / 2u) / n_buf);
        if (r == 0u)
            return false;
        const FloorPick sp = stream_select_floor<MAXW>(lkey, lnid, hist, kS, false, 0u, 0u, r,
                                                       r + r / 16u);
        const uint32_t T = uni((uint32_t)(sp.F >> 32));
        if (!sp.any || T == 0u)
            return false;
        uint32_t c = 0, mx = 0;
        for (uint32_t b = 0; b < n_buf; b += 512) {
            uint32_t kk[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t i = b + q * 64 + lane;
                kk[q] = i < n_buf ? lkey[i] : 0u;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                c += kk[q] >= T ? 1u : 0u;
                mx = kk[q] > mx ? kk[q] : mx;
            }
        }
        c = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_prefix(c), 63);
        if (c < k || c > keep_limit)
            return false;
        F = (uint64_t)T << 32;
        kmax = wave_max_u32(mx);
        return true;
    };

    // Keep the entries >= F (none if !any), in place. Eight rows of 64 per
    // step: their LDS reads overlap, and the writes of a step land below its
    // end, so nothing is overwritten before it is read. With `rebuild` the
    // histogram is rebuilt for the kept entries under the current (hb, hs).
    auto compact_to = [&](uint64_t F, bool any, bool rebuild) {
        if (rebuild) {
            *reinterpret_cast<uint4 *>(hist + lane * 4) = make_uint4(0u, 0u, 0u, 0u);
            wave_sync();
        }
        uint32_t n_new = 0;
        for (uint32_t b = 0; b < n_buf; b += 512) {
            uint32_t kk[8], nn[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t i = b + q * 64 + lane;
                kk[q] = i < n_buf ? lkey[i] : 0u;
                nn[q] = i < n_buf ? lnid[i] : 0u;
            }
            wave_sync();
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const bool keep = kk[q] != 0u && any && comp(kk[q], nn[q]) >= F;
                const uint64_t mk = __ballot(keep);
                if (keep) {
                    const uint32_t pos = n_new + lane_rank(mk);
                    lkey[pos] = kk[q];
                    lnid[pos] = nn[q];
                    if (rebuild)
                        atomicAdd(&hist[hbin(kk[q])], 1u);
                }
                n_new += (uint32_t)__popcll(mk);
            }
            wave_sync();
        }
        n_buf = uni(n_new);
    };

    auto compact = [&]() {
        wave_sync();
        if (armed) {
            // the bin holding the k-th largest key: if the entries from it up
            // number at most keep_limit, its lower edge is the new floor
            const BinHit h = wave_find_bin(hist, (int)kHB, k);
            if (h.total >= k && h.above + h.count <= keep_limit) {
                thr = uni(hb + (h.bin << hs));
                tf = key_floor_float(thr - 1u); // (blocks test their integer key)
                // the kept entries are the bins from h.bin up: while half
                // the bins remain, the histogram stays as it is, less the
                // bins below; else it is rebuilt over the narrower range
                const bool rebin = h.bin >= kHB / 2u;
                wave_sync();
                if (!rebin) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if ((uint32_t)(lane * 4 + q) < h.bin)
                            hist[lane * 4 + q] = 0u;
                } else {
                    kmax = wave_max_u32(kmax);
                    const uint32_t span = kmax - thr;
                    const uint32_t bits = span == 0u ? 0u : 32u - (uint32_t)__builtin_clz(span);
                    hs = uni(bits > 8u ? bits - 8u : 0u);
                    hb = uni(thr & ~((1u << hs) - 1u));
                }
                compact_to((uint64_t)thr << 32, true, rebin);
                return;
            }
            wave_sync();
        }
        uint64_t F = 0;
        const bool any = (!armed && sample_floor(F)) || select_floor(k, keep_limit, F);
        thr = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(F >> 32));
        // a float test admits key >= thr: a NaN floor (key 1) would have to
        // admit NaNs, which no float test does, so arming waits for a higher
        // floor
        tf = key_floor_float(thr - 1u);
        armed = STRICT ? thr != 0u : thr >= 2u;
        // bins for the keys from thr up to the largest appended so far
        const uint32_t span = kmax - thr;
        const uint32_t bits = span == 0u ? 0u : 32u - (uint32_t)__builtin_clz(span);
        hs = uni(bits > 8u ? bits - 8u : 0u);
        hb = uni(thr & ~((1u << hs) - 1u));
        compact_to(F, any, armed);
    };

    // ---- loads. Buffer loads with the hardware range check: bytes past the
    // row's end read as zero, so no load sits behind a branch.
    const __amdgpu_buffer_rsrc_t rs_row = row_rsrc(x, 0, len);
    // candidate lists are read one block id per lane per sweep, PD sweeps
    // ahead of the scores that need them
    const int32_t *cl = p.cand + (int64_t)row * p.n_cand;
    const __amdgpu_buffer_rsrc_t rs_ids =
        __builtin_amdgcn_make_buffer_rsrc((void *)cl, (short)0,
                                          MODE == MODE_CAND ? p.n_cand * 4 : 0, 0x00020000);
    auto load_id = [&](int sw) {
        // slot pair (2 * lane, 2 * lane + 1) -> one block id per lane pair
        const uint32_t c = (uint32_t)sw * (SWEEP / 8) + (uint32_t)(lane >> 1);
        return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rs_ids, (int)(c * 4u), 0, 0);
    };
    // byte offset of the half block a lane reads for candidate block id b
    auto cand_off = [&](int sw, int32_t b) {
        const uint32_t c = (uint32_t)sw * (SWEEP / 8) + (uint32_t)(lane >> 1);
        const bool ok = c < (uint32_t)p.n_cand && b >= 0 && b < (len + 7) / 8;
        return ok ? (uint32_t)b * 32u + (uint32_t)(lane & 1) * 16u : 0xfffffff0u;
    };
    // Sweep sw of the visiting order covers elements [ps * SWEEP, ps * SWEEP +
    // SWEEP) with ps = phys(sw); visits past the last sweep (the ring's
    // refills) map to nsw, past the row, where loads read nothing.
    const int nsw = (nel + SWEEP - 1) / SWEEP;
    auto phys = [&](int sw) { return sw >= nsw ? nsw : (REV ? nsw - 1 - sw : sw); };
    auto load_sweep = [&](int sw, u4 (&v)[LPS], int32_t id) {
        const int ps = phys(sw);
        if constexpr (MODE == MODE_PLAIN) {
            if constexpr (LONG)
                v[0] = load16_nt(row_rsrc(x, (int64_t)ps * SWEEP, len), (uint32_t)lane * 16u);
            else
                v[0] = load16_nt(rs_row, (uint32_t)ps * (uint32_t)(SWEEP * 4) + (uint32_t)lane * 16u);
        } else if constexpr (MODE == MODE_BLOCKS) {
            // load e covers blocks ps * 128 + e * 32 + [0, 32), 1 KiB in one
            // piece: lane l reads half (l & 1) of block e * 32 + l / 2
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (LONG) {
                    const __amdgpu_buffer_rsrc_t rs =
                        row_rsrc(x, ((int64_t)ps * SWEEP + e * 32) * 8, len);
                    v[e] = load16_nt(rs, (uint32_t)lane * 16u);
                } else {
                    const uint32_t off = ((uint32_t)ps * SWEEP + (uint32_t)(e * 32)) * 32u +
                                         (uint32_t)lane * 16u;
                    v[e] = load16_nt(rs_row, off);
                }
            }
        } else {
            v[0] = load16_nt(rs_row, cand_off(sw, id));
        }
    };

    // ---- one sweep's elements: raw score bits (blocks: their key, absent
    // candidates: a NaN, which fails every test) and ~index. Validity against
    // the row's end is checked only in TAIL sweeps, the ones that reach it.
    struct Elem {
        uint32_t val[EPL];
        uint32_t nid[EPL];
        bool ok[EPL]; // candidates: the slot holds a position of the row
    };
    auto decode = [&](const u4 (&v)[LPS], int sw, int32_t id, auto tail) {
        constexpr bool TAIL = decltype(tail)::value;
        const int ps = phys(sw);
        Elem el;
        if constexpr (MODE == MODE_PLAIN) {
            const int32_t i0 = ps * SWEEP + lane * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                el.val[e] = v[0][e];
                el.nid[e] = ~(uint32_t)(i0 + e);
            }
        } else if constexpr (MODE == MODE_BLOCKS) {
            // Best raw key of each half block (the key map without its -0.0
            // and NaN fix-ups: two operations per score), the two halves of a
            // block combined across the lane pair; a lane then keeps the
            // blocks of loads (l & 1) and (l & 1) + 2, the fix-ups applied
            // once per block.
            const int h = lane & 1;
            uint32_t pm[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int32_t p0 = (ps * SWEEP + e * 32 + (lane >> 1)) * 8 + h * 4;
                uint32_t b = 0u;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    b = max(b, (!TAIL || p0 + j < len) ? raw_key(v[e][j]) : 0u);
                pm[e] = max(b, dpp<0xB1, 0xf>(b, 0u)); // quad_perm [1,0,3,2]: the pair
            }
            bool nan_pos = false;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                nan_pos = nan_pos || pm[e] > 0xff800000u;
            if (__ballot(nan_pos) != 0ull) {
                // a positive NaN outranks everything under the raw map: score
                // the wave's blocks exactly (rare; every lane takes part, as
                // the halves combine across lanes)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int32_t p0 = (ps * SWEEP + e * 32 + (lane >> 1)) * 8 + h * 4;
                    uint32_t b = 0u;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        b = max(b, (!TAIL || p0 + j < len) ? score_key(v[e][j]) : 0u);
                    const uint32_t x2 = max(b, dpp<0xB1, 0xf>(b, 0u));
                    pm[e] = pm[e] > 0xff800000u ? x2 : pm[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                uint32_t best = h ? pm[2 * e + 1] : pm[2 * e];
                const int32_t blk = ps * SWEEP + (2 * e + h) * 32 + (lane >> 1);
                if (best == 0x7fffffffu)
                    best = 0x80000000u; // the best score is -0.0
                else if (best < 0x007fffffu && blk < nel)
                    best = 1u;          // only negative NaNs (raw keys below -inf's)
                el.val[e] = best; // 0 (absent) for blocks past the end
                el.nid[e] = ~(uint32_t)blk;
            }
        } else {
            const uint32_t off = cand_off(sw, id);
            const int32_t p0 = (int32_t)(off >> 2);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                el.ok[e] = off != 0xfffffff0u && p0 + e < len;
                el.val[e] = el.ok[e] ? v[0][e] : 0x7fc00000u;
                el.nid[e] = ~(uint32_t)(p0 + e);
            }
        }
        return el;
    };
    // valid element (plain rows: inside the row; blocks: key 0 means none
    // of its positions is; candidates: flagged by decode)
    auto valid = [&](const Elem &el, int sw, int e) {
        if constexpr (MODE == MODE_PLAIN)
            return phys(sw) * SWEEP + lane * 4 + e < len;
        else if constexpr (MODE == MODE_BLOCKS)
            return el.val[e] != 0u;
        else
            return el.ok[e];
    };
    auto test = [&](uint32_t val) {
        return MODE == MODE_BLOCKS ? val > thr : __uint_as_float(val) >= tf;
    };

    // One sweep (every branch is on wave-uniform values).
    auto sweep_body = [&](const u4 (&v)[LPS], int sw, int32_t id, auto tail) {
        constexpr bool TAIL = decltype(tail)::value;
        const Elem el = decode(v, sw, id, tail);
        if (!armed) {
            uint32_t kq[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const uint32_t kk = MODE == MODE_BLOCKS ? el.val[e] : score_key(el.val[e]);
                // plain rows are valid throughout a sweep that ends inside the row
                kq[e] = (MODE == MODE_PLAIN && !TAIL) || valid(el, sw, e) ? kk : 0u;
            }
            if constexpr (EPL == 4) {
                if ((n_buf & 3u) == 0u) {
                    // 16-byte writes need n_buf % 4 == 0 (always so before the
                    // first compaction)
                    *reinterpret_cast<uint4 *>(lkey + n_buf + lane * 4) =
                        make_uint4(kq[0], kq[1], kq[2], kq[3]);
                    *reinterpret_cast<uint4 *>(lnid + n_buf + lane * 4) =
                        make_uint4(el.nid[0], el.nid[1], el.nid[2], el.nid[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        lkey[n_buf + lane * 4 + e] = kq[e];
                        lnid[n_buf + lane * 4 + e] = el.nid[e];
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    lkey[n_buf + e * 64 + lane] = kq[e];
                    lnid[n_buf + e * 64 + lane] = el.nid[e];
                }
            }
            n_buf += SWEEP;
            return;
        }
        // armed: one test per element; the masks are reused for the appends
        uint64_t m[EPL];
        uint64_t any = 0ull;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            m[e] = __ballot(test(el.val[e]));
            any |= m[e];
        }
        if (any == 0ull)
            return;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            if (m[e] != 0ull) {
                bool pass = test(el.val[e]);
                // plain rows: bytes past the row's end read as +0.0, which may pass
                if (TAIL && MODE == MODE_PLAIN)
                    pass = pass && valid(el, sw, e);
                const uint64_t mk = TAIL && MODE == MODE_PLAIN ? __ballot(pass) : m[e];
                if (pass) {
                    // +0.0f turns -0.0 into +0.0, the key both zeros share
                    const uint32_t kk =
                        MODE == MODE_BLOCKS
                            ? el.val[e]
                            : raw_key(__float_as_uint(__uint_as_float(el.val[e]) + 0.0f));
                    const uint32_t pos = n_buf + lane_rank(mk);
                    lkey[pos] = kk;
                    lnid[pos] = el.nid[e];
                    atomicAdd(&hist[hbin(kk)], 1u);
                    kmax = kk > kmax ? kk : kmax;
                }
                n_buf = uni(n_buf + (uint32_t)__popcll(mk));
            }
        }
    };
    auto process = [&](const u4 (&v)[LPS], int sw, int32_t id) {
        if (sw >= nsw)
            return;
        const int32_t base = phys(sw) * SWEEP;
        // sweeps that reach the row's end (blocks: its last, partial block)
        const bool tail = MODE == MODE_BLOCKS ? (int64_t)(base + SWEEP) * 8 > len
                                              : base + SWEEP > nel;
        if (tail)
            sweep_body(v, sw, id, std::true_type{});
        else
            sweep_body(v, sw, id, std::false_type{});
    };

    // ---- the ring of PD sweeps in flight. A scheduling barrier after each
    // stage's refill keeps the refill behind that stage's work.
    u4 buf[PD][LPS];
    int32_t idr[PD];   // candidates: block id for the sweep PD ahead of the stage
    int32_t idc[PD];   // candidates: block id of the sweep in buf[d]
#pragma unroll
    for (int d = 0; d < PD; ++d)
        idc[d] = MODE == MODE_CAND ? load_id(d) : 0;
#pragma unroll
    for (int d = 0; d < PD; ++d) {
        load_sweep(d, buf[d], idc[d]);
        idr[d] = MODE == MODE_CAND ? load_id(d + PD) : 0;
        __builtin_amdgcn_sched_barrier(0);
    }
    // Memory arbitration favours the oldest waves on a SIMD, so rows that
    // start later fall behind and stretch the end of a launch. A wave's
    // priority falls as its row progresses (3 in the first quarter, 0 in the
    // last), so the rows furthest behind issue first. (The block stage runs
    // one wave per SIMD, where priorities decide nothing.)
    constexpr bool PRIO = MODE != MODE_BLOCKS;
    int quarter = 0;
    if (PRIO)
        __builtin_amdgcn_s_setprio(3);
    for (int s0 = 0; s0 < nsw; s0 += PD) {
        if (PRIO && quarter < 3 && s0 * 4 >= nsw * (quarter + 1)) {
            ++quarter;
            if (quarter == 1)
                __builtin_amdgcn_s_setprio(2);
            else if (quarter == 2)
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
        }
#pragma unroll
        for (int d = 0; d < PD; ++d) {
            process(buf[d], s0 + d, idc[d]);
            load_sweep(s0 + d + PD, buf[d], idr[d]);
            if constexpr (MODE == MODE_CAND) {
                idc[d] = idr[d];
                idr[d] = load_id(s0 + d + 2 * PD);
            }
            if (n_buf > (uint32_t)CAPS)
                compact();
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- final exact selection over the buffer. With the histogram: the
    // entries of the bins above the k-th largest's bin are written out as
    // they are met, the ones of that bin (if at most 64) staged in the
    // histogram's words and ranked one per lane. Otherwise (or if the stage
    // finds no unique rank) radix select gives the floor composite F and
    // every entry >= F is written out.
    wave_sync();
    bool done = false, pre = false;
    uint64_t pre_F = 0;
    if (n_buf > k && armed) {
        const BinHit h = wave_find_bin(hist, (int)kHB, k);
        wave_sync();
        if (h.total >= k && h.count <= 64u) {
            const uint32_t need = k - h.above; // 1 <= need <= h.count
            uint32_t n_out = 0, ns = 0;
            for (uint32_t b = 0; b < n_buf; b += 512) {
                uint32_t kk[8], nn[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint32_t i = b + q * 64 + lane;
                    kk[q] = i < n_buf ? lkey[i] : 0u;
                    nn[q] = i < n_buf ? lnid[i] : 0u;
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const bool live = b + q * 64 + lane < n_buf;
                    const uint32_t bn = hbin(kk[q]);
                    const bool top = live && bn > h.bin;
                    const bool in = live && bn == h.bin;
                    const uint64_t mt = __ballot(top);
                    const uint64_t mi = __ballot(in);
                    const uint32_t pt = n_out + lane_rank(mt);
                    const uint32_t pi = ns + lane_rank(mi);
                    if (top && pt < k)
                        out[pt] = (int32_t)~nn[q];
                    if (in && pi < 64u) {
                        hist[pi] = kk[q];
                        hist[64 + pi] = nn[q];
                    }
                    n_out += (uint32_t)__popcll(mt);
                    ns += (uint32_t)__popcll(mi);
                }
            }
            wave_sync();
            const uint32_t nb = ns < 64u ? ns : 64u;
            const uint64_t mine = (uint32_t)lane < nb ? comp(hist[lane], hist[64 + lane]) : 0ull;
            uint32_t r = 0;
            for (uint32_t j = 0; j < nb; ++j) {
                const uint32_t olo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine, (int)j);
                const uint32_t ohi =
                    (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mine >> 32), (int)j);
                r += (((uint64_t)ohi << 32) | olo) > mine ? 1u : 0u;
            }
            const bool win = (uint32_t)lane < nb && r < need;
            const uint64_t mw = __ballot(win);
            // the bin's entries are distinct composites unless candidate
            // ids repeat: then the ranks tie and the counts disagree
            if (n_out == h.above && ns == h.count && (uint32_t)__popcll(mw) == need) {
                if (win)
                    out[n_out + lane_rank(mw)] = (int32_t)~(uint32_t)mine;
                done = true;
            }
            wave_sync();
        } else if (h.total >= k && h.bin < kHB - 1u) {
            // a larger bin below the top one: its keys share one prefix, so
            // radix select starts from it
            SelState st;
            st.s = 32 + (int)hs;
            st.P = (uint64_t)((hb >> hs) + h.bin);
            st.above = h.above;
            st.cnt = h.count;
            st.need = k - h.above;
            wave_lds_select<MAXW>(lkey, lnid, n_buf, st, hist, 0u);
            pre_F = sel_floor(st);
            pre = true;
        }
    }
    if (!done) {
        __threadfence_block(); // after any writes of an abandoned attempt
        uint64_t F = pre_F;
        const bool any = n_buf <= k || pre ? true : select_floor(k, 0u, F);
        uint32_t n_out = 0;
        for (uint32_t b = 0; b < n_buf; b += 512) {
            uint32_t kk[8], nn[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t i = b + q * 64 + lane;
                kk[q] = i < n_buf ? lkey[i] : 0u;
                nn[q] = i < n_buf ? lnid[i] : 0u;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const bool keep = kk[q] != 0u && any && comp(kk[q], nn[q]) >= F;
                const uint64_t mk = __ballot(keep);
                const uint32_t pos = n_out + lane_rank(mk);
                if (keep && pos < k) // (repeated candidate ids could exceed k)
                    out[pos] = (int32_t)~nn[q];
                n_out += (uint32_t)__popcll(mk);
            }
        }
        for (uint32_t i = (n_out < k ? n_out : k) + lane; i < k; i += 64)
            out[i] = -1;
    }
}

// ------------------------------------------------------------------ row kernel

// Whole rows of up to T * E scores, one workgroup per row and no exchange
// between workgroups (decode batches: many rows of up to 32,768). With 16
// waves per CU every instruction is paid sixteen times per SIMD, so a thread
// keeps its E scores exactly as loaded (E/4 vectors: positions
// (g * T + t) * 4 + [0, 4)) and touches each with a couple of instructions:
//   1. each thread's largest valid score (float max: NaNs drop out, and a
//      thread whose valid scores are all NaN has a NaN max) goes into a 12-bit
//      histogram of keys; the bin where m = min(k, len) maxima are reached from
//      the top has at least m scores at or above its lower edge B, so every
//      score below B is out;
//   2. each thread marks the scores at or above B in a bit mask (one float
//      compare each; about 2 % of an i.i.d. row), one block-wide scan places
//      them, the row's scores are staged in LDS by position, and each thread
//      walks its mask's set bits only, writing (key, ~index) to a list;
//   3. the list is loaded back, two per thread, and an exact radix select
//      finishes the row.
// Rows with fewer maxima than m keep every valid score; more than CAP
// survivors (heavy ties, rows that rise everywhere) fall back to the exact
// digit-by-digit selection over the row re-read from memory.
template <int T, int E>
__global__ __launch_bounds__(T) void row_kernel(KParams p)
{
    constexpr int NV = E / 4;
    constexpr int MAXW = 12;
    constexpr int NB = HistBuf<MAXW>::NB;
    constexpr int CAP = 2 * T;
    static_assert(E % 4 == 0 && E <= 32, "one 32-bit mask per thread");
    static_assert(T * E >= 3 * NB, "the staged row holds the select's histograms afterwards");
    // the row's scores by position, then the register select's histograms
    __shared__ __attribute__((aligned(16))) uint32_t stage[T * E];
    // the bound's histogram, then the survivor list (keys, then ~indices)
    __shared__ __attribute__((aligned(16))) uint32_t lst[NB];
    __shared__ uint32_t tmp[T / 64];
    __shared__ uint32_t res[4];
    __shared__ uint32_t ctr;
    __shared__ uint32_t kmax; // the row's largest key
    static_assert(2 * CAP <= NB, "the list fits the histogram's words");

    const int row = p.row0 + (int)blockIdx.x;
    const int32_t len = row_len(p, row);
    const uint32_t k = (uint32_t)p.k;
    const uint32_t m = (uint32_t)len < k ? (uint32_t)len : k;
    int32_t *out = p.out + (int64_t)row * p.k;
    const float *x = p.scores + (int64_t)row * p.row_stride;
    const int t = threadIdx.x;

    if ((uint32_t)len <= k) {
        // every valid position is selected
        for (uint32_t i = (uint32_t)t; i < k; i += T)
            out[i] = i < (uint32_t)len ? (int32_t)i : -1;
        return;
    }
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(x, 0, len);
    u4 f[NV];
#pragma unroll
    for (int g = 0; g < NV; ++g)
        f[g] = load16(rs, (uint32_t)(g * T + t) * 16u);
    block_zero<T>(lst, NB);
    if (t == 0)
        kmax = 0u;
    // Positions (g * T + t) * 4 + j. Vectors below gv hold valid scores for
    // every thread; vector gv is partial, the ones above it empty. The
    // branches on g are uniform, so only the partial vector pays for masks.
    const int gv = len / (4 * T);
    auto pos = [&](int g, int j) { return (g * T + t) * 4 + j; };
    const float qnan = __uint_as_float(0x7fc00000u);
    float fm = qnan;
#pragma unroll
    for (int g = 0; g < NV; ++g) {
        const float a0 = __uint_as_float(f[g][0]), a1 = __uint_as_float(f[g][1]);
        const float a2 = __uint_as_float(f[g][2]), a3 = __uint_as_float(f[g][3]);
        if (g < gv) {
            fm = __builtin_fmaxf(fm, __builtin_fmaxf(a0, a1));
            fm = __builtin_fmaxf(fm, __builtin_fmaxf(a2, a3));
        } else if (g == gv) {
            fm = __builtin_fmaxf(fm, pos(g, 0) < len ? a0 : qnan);
            fm = __builtin_fmaxf(fm, pos(g, 1) < len ? a1 : qnan);
            fm = __builtin_fmaxf(fm, pos(g, 2) < len ? a2 : qnan);
            fm = __builtin_fmaxf(fm, pos(g, 3) < len ? a3 : qnan);
        }
    }
    // (+0.0f turns a -0.0 maximum into +0.0; a NaN maximum -- all the
    // thread's valid scores NaN -- maps to key 1)
    const bool any = pos(0, 0) < len;
    const uint32_t tkey = any ? score_key(__float_as_uint(fm + 0.0f)) : 0u;
    __syncthreads();
    if (tkey != 0u)
        atomicAdd(&lst[tkey >> 20], 1u);
    {
        const uint32_t wm = wave_max_u32(tkey);
        if ((t & 63) == 0)
            atomicMax(&kmax, wm);
    }
    __syncthreads();
    const BinHit th = block_find_bin<T>(lst, NB, m, tmp, res);
    // Lower edge of the bound's bin, as a float test: key(x) >= B <=> x >= fb.
    // With fewer maxima than m (rows shorter than 4 m), or a bound in the
    // lowest bin (NaN keys reach it, which no float test admits), every valid
    // score is kept.
    const uint32_t B = th.total >= m ? (th.bin << 20) : 0u;
    const bool all = B == 0u;
    const float fb = all ? -__builtin_inff() : key_floor_float(B - 1u);
    // bit 4 g + j: score (g, j) kept -- valid and (all or x >= fb); NaNs pass
    // only with `all` (bitwise operators: short-circuit forms become branches)
    uint32_t mask = 0;
#pragma unroll
    for (int g = 0; g < NV; ++g) {
        if (g <= gv) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = __uint_as_float(f[g][j]);
                const int ok = (int)(g < gv) | (int)(pos(g, j) < len);
                const int kp = ok & ((int)(v >= fb) | (int)all);
                mask |= (uint32_t)kp << (4 * g + j);
            }
        }
    }
    uint32_t tot;
    uint32_t at = block_excl_prefix<T>((uint32_t)__popc(mask), tmp, tot);
    if (tot > (uint32_t)CAP) {
        if (t == 0)
            ctr = 0u;
        __syncthreads();
        block_row_select<T, 8, MODE_PLAIN, MAXW>(p, row, len, (uint32_t)len, m, out, lst, tmp,
                                                  res, &ctr);
        for (uint32_t i = m + (uint32_t)t; i < k; i += T)
            out[i] = -1;
        return;
    }
    // the row by position in LDS (the survivors are read back from there; the
    // list overwrites the bound's histogram, last read by the find-bin)
#pragma unroll
    for (int g = 0; g < NV; ++g)
        if (g <= gv)
            *reinterpret_cast<u4 *>(stage + (g * T + t) * 4) = f[g];
    __syncthreads();
    while (mask != 0u) {
        const int bit = __builtin_ctz(mask);
        mask &= mask - 1u;
        const int ps = ((bit >> 2) * T + t) * 4 + (bit & 3);
        lst[at] = score_key(stage[ps]);
        lst[CAP + at] = ~(uint32_t)ps;
        ++at;
    }
    __syncthreads();
    uint32_t sk[2], sn[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const uint32_t i = (uint32_t)t + (uint32_t)u * T;
        sk[u] = i < tot ? lst[i] : 0u;
        sn[u] = i < tot ? lst[CAP + i] : 0u;
    }
    // the staged row's words become the select's three histograms
    block_zero<T>(stage, 2 * NB);
    __syncthreads();
    // every survivor lies in [B, the row's largest key]: the select starts
    // below the bits those share (often one digit pass fewer)
    SelState st = sel_start_range((uint64_t)B << 32, ((uint64_t)kmax << 32) | 0xffffffffull, tot, m);
    block_regs_select<T, MAXW>(sk, sn, st, 0u, stage, tmp, res, index_bits((int64_t)len));
    const uint64_t F = sel_floor(st);
    const uint32_t fk = (uint32_t)(F >> 32), fn = (uint32_t)F;
    uint32_t ns = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u)
        ns += at_or_above(sk[u], sn[u], fk, fn) ? 1u : 0u;
    uint32_t tt;
    uint32_t slot = block_excl_prefix<T>(ns, tmp, tt);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (at_or_above(sk[u], sn[u], fk, fn)) {
            if (slot < m)
                out[slot] = (int32_t)~sn[u];
            ++slot;
        }
    }
    for (uint32_t i = m + (uint32_t)t; i < k; i += T)
        out[i] = -1;
}

// Candidate lists of blocks of eight (the shared-candidate layer's second
// stage), up to 2 T blocks per row: one workgroup per row, as row_kernel. A
// thread gathers its two blocks (slots t and t + T of the list: four 16-byte
// loads; an id outside the row reads nothing) and keeps the 16 scores as
// loaded; the bound comes from the thread maxima, the scores at or above it
// are marked, staged by slot in LDS and walked into a list of (key,
// ~position) that an exact radix select finishes, two per thread. More than
// CAP survivors fall back to the digit-by-digit selection over the list
// re-read from memory. Repeated ids leave the result undefined, as
// everywhere.
// The candidate row's work for row `row`, by one workgroup of T threads. LDS:
// stage[T * 16] (the gathered scores by slot, vector v of thread t at
// (v T + t) 4, then the register select's histograms), lst[4096] (the bound's
// histogram, then the survivor list: keys, then ~positions), tmp[T / 64],
// res[4], and three words sm: a counter, the row's largest candidate key, the
// valid candidate count. The caller has the workgroup past a barrier.
template <int T>
__device__ void cand_rows_finish(const KParams &p, int row, uint32_t *stage, uint32_t *lst,
                                 uint32_t *tmp, uint32_t *res, uint32_t *sm)
{
    constexpr int E = 16;
    constexpr int MAXW = 12;
    constexpr int NB = HistBuf<MAXW>::NB;
    constexpr int CAP = 2 * T;
    static_assert(T * E >= 3 * NB && 2 * CAP <= NB, "LDS reuse");
    uint32_t &ctr = sm[0], &kmax = sm[1], &vcnt = sm[2];

    const int32_t len = row_len(p, row);
    const uint32_t k = (uint32_t)p.k;
    int32_t *out = p.out + (int64_t)row * p.k;
    const float *x = p.scores + (int64_t)row * p.row_stride;
    const int32_t *cl = p.cand + (int64_t)row * p.n_cand;
    const int t = threadIdx.x;

    int32_t lo[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int slot = g * T + t;
        const int64_t b = slot < p.n_cand ? (int64_t)cl[slot] : -1;
        lo[g] = (b >= 0 && b * 8 < (int64_t)len) ? (int32_t)(b * 8) : -1;
    }
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(x, 0, len);
    u4 f[4];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        // an id outside the row reads past the range: zeros, no access
        const uint32_t off = lo[g] >= 0 ? (uint32_t)lo[g] * 4u : 0xfffffff0u;
        f[2 * g] = load16(rs, off);
        f[2 * g + 1] = load16(rs, off + 16u);
    }
    block_zero<T>(lst, NB);
    if (t == 0) {
        kmax = 0u;
        vcnt = 0u;
    }
    // valid scores: bit 8 g + i (i = 4 h + j for vector 2 g + h)
    uint32_t vm = 0;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            vm |= (uint32_t)(lo[g] >= 0 && lo[g] + i < len) << (8 * g + i);
    const float qnan = __uint_as_float(0x7fc00000u);
    float fm = qnan;
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            fm = __builtin_fmaxf(fm, (vm >> (4 * v + j)) & 1u ? __uint_as_float(f[v][j]) : qnan);
    const uint32_t tkey = vm != 0u ? score_key(__float_as_uint(fm + 0.0f)) : 0u;
    __syncthreads();
    if (tkey != 0u)
        atomicAdd(&lst[tkey >> 20], 1u);
    {
        const uint32_t wm = wave_max_u32(tkey);
        const uint32_t wv = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_prefix((uint32_t)__popc(vm)), 63);
        if ((t & 63) == 0) {
            atomicMax(&kmax, wm);
            atomicAdd(&vcnt, wv);
        }
    }
    __syncthreads();
    const uint32_t V = uni(vcnt);
    const uint32_t m = V < k ? V : k;
    if (m == 0u) {
        for (uint32_t i = (uint32_t)t; i < k; i += T)
            out[i] = -1;
        return;
    }
    const BinHit th = block_find_bin<T>(lst, NB, m, tmp, res);
    // Every valid score is kept when the bound cannot be found (m or fewer
    // thread maxima) or lies in the lowest bin (NaN keys reach it).
    const uint32_t B = th.total >= m ? (th.bin << 20) : 0u;
    const bool all = B == 0u;
    const float fb = all ? -__builtin_inff() : key_floor_float(B - 1u);
    uint32_t mask = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int bit = 4 * v + j;
            const int kp = (int)((vm >> bit) & 1u) & ((int)(__uint_as_float(f[v][j]) >= fb) | (int)all);
            mask |= (uint32_t)kp << bit;
        }
    uint32_t tot;
    uint32_t at = block_excl_prefix<T>((uint32_t)__popc(mask), tmp, tot);
    if (tot > (uint32_t)CAP) {
        if (t == 0)
            ctr = 0u;
        __syncthreads();
        block_row_select<T, 8, MODE_CAND, MAXW>(p, row, len, V, m, out, lst, tmp, res, &ctr);
        for (uint32_t i = m + (uint32_t)t; i < k; i += T)
            out[i] = -1;
        return;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
        *reinterpret_cast<u4 *>(stage + (v * T + t) * 4) = f[v];
    __syncthreads();
    while (mask != 0u) {
        const int bit = __builtin_ctz(mask);
        mask &= mask - 1u;
        const int32_t base = (bit >> 3) != 0 ? lo[1] : lo[0];
        lst[at] = score_key(stage[((bit >> 2) * T + t) * 4 + (bit & 3)]);
        lst[CAP + at] = ~(uint32_t)(base + (bit & 7));
        ++at;
    }
    __syncthreads();
    uint32_t sk[2], sn[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const uint32_t i = (uint32_t)t + (uint32_t)u * T;
        sk[u] = i < tot ? lst[i] : 0u;
        sn[u] = i < tot ? lst[CAP + i] : 0u;
    }
    block_zero<T>(stage, 2 * NB);
    __syncthreads();
    SelState st = sel_start_range((uint64_t)B << 32, ((uint64_t)kmax << 32) | 0xffffffffull, tot, m);
    block_regs_select<T, MAXW>(sk, sn, st, 0u, stage, tmp, res, index_bits((int64_t)p.n_max));
    const uint64_t F = sel_floor(st);
    const uint32_t fk = m != 0u ? (uint32_t)(F >> 32) : 0xffffffffu;
    const uint32_t fn = m != 0u ? (uint32_t)F : 0xffffffffu;
    uint32_t ns = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u)
        ns += at_or_above(sk[u], sn[u], fk, fn) ? 1u : 0u;
    uint32_t tt;
    uint32_t slot = block_excl_prefix<T>(ns, tmp, tt);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (at_or_above(sk[u], sn[u], fk, fn)) {
            if (slot < m)
                out[slot] = (int32_t)~sn[u];
            ++slot;
        }
    }
    for (uint32_t i = m + (uint32_t)t; i < k; i += T)
        out[i] = -1;
}

template <int T>
__global__ __launch_bounds__(T) void cand_row_kernel(KParams p)
{
    __shared__ __attribute__((aligned(16))) uint32_t stage[T * 16];
    __shared__ __attribute__((aligned(16))) uint32_t lst[HistBuf<12>::NB];
    __shared__ uint32_t tmp[T / 64];
    __shared__ uint32_t res[4];
    __shared__ uint32_t sm[3];
    cand_rows_finish<T>(p, p.row0 + (int)blockIdx.x, stage, lst, tmp, res, sm);
}

__global__ void empty_kernel() {}

// ---------------------------------------------------- launch configuration

constexpr int kSplitT = 1024;
// Elements per thread of the split kernel. Plain rows and the block stage take
// the smallest of a mode's choices whose grid still fits the device in one
// round (more, smaller chunks shorten each workgroup's load and local
// selection), else the largest. Candidate lists that one workgroup holds (8
// or 16 slots per thread) are selected whole, with no exchange; longer lists
// are split in chunks of 8 slots per thread.
constexpr int kPlainE = 8;   // 8192 scores per workgroup
constexpr int kPlainEFine = 4;
constexpr int kBlocksE = 4;  // 4096 blocks per workgroup
constexpr int kBlocksEFine = 1;
constexpr int kCandE = 8;    // 8192 candidate slots per workgroup
constexpr int kCandEWhole = 16; // lists of up to 16384 slots (2048 blocks of 8) in one workgroup
// Streaming kernel: sweeps in flight per wave. Plain rows 16 (a sweep is one
// 16-byte load per lane); the block stage 4 (four loads per sweep);
// candidates 8 (one load plus the block ids it needs, fewer registers).
template <int MODE>
constexpr int stream_pd()
{
    return MODE == MODE_PLAIN ? 16 : (MODE == MODE_BLOCKS ? 4 : 8);
}
constexpr int kStreamMaxW = 8;
// Buffer slots per k range: a compaction above BUF - SWEEP (at least 1.5k)
// keeps a little over k, freeing a quarter of the buffer or more. The small
// buffer (9 KiB of LDS with the histogram) lets 16 waves share a CU, which
// plain rows need more than they need fewer compactions.
constexpr int kStreamBuf512 = 1024;
constexpr int kStreamBuf1024 = 2048;
constexpr int kStreamBuf2048 = 4096;
constexpr int kStreamBuf4096 = 8192;

// ------------------------------------------------------------------ host side


// Built-in workspace of lt_topk_run_noalloc: the row records of up to
// kNoAllocRows split rows. Each GPU the library runs on holds its own copy
// until the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in, not a device address).
constexpr int kNoAllocRows = 64;
constexpr size_t kNoAllocBytes = (size_t)kNoAllocRows * kWsRowWords * 4; // 5,193,728
static __device__ __align__(256) uint32_t scratch[(size_t)kNoAllocRows * kWsRowWords];
static_assert(kNoAllocRows == LT_NOALLOC_SPLIT_ROWS && kNoAllocBytes == LT_NOALLOC_BYTES,
              "the header states the built-in workspace's size");

struct DeviceInfo {
    bool ready;
    int cus;
    uint32_t *scratch_ptr;              // this device's copy of `scratch`
    std::atomic<bool> *scratch_pending; // its tickets still need clearing
};

static std::mutex g_mu;
static DeviceInfo g_dev[64];
static std::atomic<bool> g_scratch_pending[64];
// Test hooks (ltopk_debug.h). Atomic so that a hook set on one thread while
// another launches is a well-defined read of either the old or the new value.
static std::atomic<int> g_force_path{0};     // 0 auto, 1 split, 2 stream (rows without candidates)
static std::atomic<int> g_force_fallback{0}; // 1: split rows always take the exact re-read path
static std::atomic<int> g_force_sample{0};   // 0 mode word, 1 never sample, 2 always sample

static hipError_t device_info(DeviceInfo &out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= 64)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceInfo &d = g_dev[dev];
    if (!d.ready) {
        e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
        // once per device, with that device current: the address of its copy
        // of the built-in workspace (lt_topk_run_noalloc)
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        d.scratch_ptr = static_cast<uint32_t *>(ptr);
        g_scratch_pending[dev].store(true);
        d.scratch_pending = &g_scratch_pending[dev];
        d.ready = true;
    }
    out = d;
    return hipSuccess;
}

// Zeroes the ticket and mode words of each row record of a built-in
// workspace: the parts of it that must start at zero (every call returns the
// tickets it used to zero). A kernel rather than a memset, so that a call
// under stream capture records an ordinary kernel node.
__global__ void clear_tickets_kernel(uint32_t *ws, int rows)
{
    const int r = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (r < rows) {
        ws[(int64_t)r * kWsRowWords + kWsTicket] = 0u;
        ws[(int64_t)r * kWsRowWords + kWsMode] = 0u;
    }
}

// The workspace a call's split rows use: the caller's (pending == nullptr), or
// a built-in one whose tickets are cleared before the first split launch that
// uses it. The flag drops only when that clearing was enqueued outside stream
// capture; a captured clearing becomes part of the graph, and the next call
// outside capture clears again.
struct WsArg {
    size_t bytes;
    std::atomic<bool> *pending;
};

template <int E, int MODE, bool WHOLE = false>
static lt_status launch_split(KParams p, int32_t B, int64_t vlen, const WsArg &wa,
                              hipStream_t stream)
{
    constexpr int64_t C = (int64_t)kSplitT * E;
    const int64_t S = vlen > 0 ? (vlen + C - 1) / C : 1;
    if (S > kMaxS || (WHOLE && S != 1))
        return LT_EINVAL;
    p.vlen = vlen;
    p.force_fallback = (uint32_t)g_force_fallback.load(std::memory_order_relaxed);
    p.force_sample = (uint32_t)g_force_sample.load(std::memory_order_relaxed);
    int64_t rows_per = 65535;
    if (S > 1) {
        rows_per = B < kMaxSplitRows ? B : kMaxSplitRows;
        if (p.ws == nullptr || wa.bytes < (size_t)rows_per * kWsRowWords * 4)
            return LT_ENOSPC;
        if (wa.pending != nullptr && wa.pending->load()) {
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            if (hipStreamIsCapturing(stream, &cs) != hipSuccess)
                return LT_EHIP;
            hipLaunchKernelGGL(clear_tickets_kernel, dim3((kNoAllocRows + 63) / 64), dim3(64), 0,
                               stream, p.ws, kNoAllocRows);
            if (cs == hipStreamCaptureStatusNone)
                wa.pending->store(false);
        }
    }
    for (int32_t r0 = 0; r0 < B; r0 += (int32_t)rows_per) {
        const int32_t rows = (int32_t)(B - r0 < rows_per ? B - r0 : rows_per);
        KParams q = p;
        q.row0 = r0;
        hipLaunchKernelGGL((split_kernel<kSplitT, E, MODE, WHOLE>), dim3((unsigned)S, rows),
                           dim3(kSplitT), 0, stream, q);
    }
    return hipGetLastError() == hipSuccess ? LT_OK : LT_EHIP;
}

// Rows up to this many scores are read through one buffer resource per row.
constexpr int32_t kStreamShortMax = (1 << 29) - 4096;

template <int MODE, int BUF>
static void launch_stream_buf(const KParams &q, int32_t rows, hipStream_t stream)
{
    if (q.n_max <= kStreamShortMax)
        hipLaunchKernelGGL((stream_kernel<MODE, BUF, stream_pd<MODE>(), kStreamMaxW, false>), dim3(rows),
                           dim3(64), 0, stream, q);
    else
        hipLaunchKernelGGL((stream_kernel<MODE, BUF, stream_pd<MODE>(), kStreamMaxW, true>), dim3(rows),
                           dim3(64), 0, stream, q);
}

template <int MODE>
static lt_status launch_stream(KParams p, int32_t B, hipStream_t stream)
{
    for (int32_t r0 = 0; r0 < B; r0 += 1 << 30) {
        KParams q = p;
        q.row0 = r0;
        const int32_t rows = B - r0 < (1 << 30) ? B - r0 : (1 << 30);
        if (p.k <= 512)
            launch_stream_buf<MODE, kStreamBuf512>(q, rows, stream);
        else if (p.k <= 1024)
            launch_stream_buf<MODE, kStreamBuf1024>(q, rows, stream);
        else if (p.k <= 2048)
            launch_stream_buf<MODE, kStreamBuf2048>(q, rows, stream);
        else
            launch_stream_buf<MODE, kStreamBuf4096>(q, rows, stream);
    }
    return hipGetLastError() == hipSuccess ? LT_OK : LT_EHIP;
}

// Whole rows in one workgroup each (row_kernel): rows of more than one split
// chunk's 4096 scores and up to 32,768. (Measured against the split kernel
// for 1 to 256 rows of 8192 to 32,768 scores: faster at every size, from
// 10.3 to 9.2 us for one row of 32,768 to 43.9 to 11.1 us for 256.)
constexpr int kRowT = 1024;
constexpr int kRowE = 32;
constexpr int32_t kRowMax = kRowT * kRowE; // 32,768

static lt_status launch_rows(KParams p, int32_t B, hipStream_t stream)
{
    for (int32_t r0 = 0; r0 < B; r0 += 1 << 30) {
        KParams q = p;
        q.row0 = r0;
        const int32_t rows = B - r0 < (1 << 30) ? B - r0 : (1 << 30);
        hipLaunchKernelGGL((row_kernel<kRowT, kRowE>), dim3(rows), dim3(kRowT), 0, stream, q);
    }
    return hipGetLastError() == hipSuccess ? LT_OK : LT_EHIP;
}

// Candidate lists of up to 2048 blocks of eight, one workgroup per row
// (cand_row_kernel). Measured against the whole-list split kernel: 8.8
// against 9.4 us for one row, 9.0 against 11.2 us for 32; for the 8192 rows
// of a prefill batch the streaming kernel stays ahead (0.31 against 0.49 ms),
// so batches past four rows per CU stream.
static lt_status launch_cand_rows(KParams p, int32_t B, hipStream_t stream)
{
    p.vlen = (int64_t)p.n_cand * p.bs;
    for (int32_t r0 = 0; r0 < B; r0 += 1 << 30) {
        KParams q = p;
        q.row0 = r0;
        const int32_t rows = B - r0 < (1 << 30) ? B - r0 : (1 << 30);
        hipLaunchKernelGGL((cand_row_kernel<kRowT>), dim3(rows), dim3(kRowT), 0, stream, q);
    }
    return hipGetLastError() == hipSuccess ? LT_OK : LT_EHIP;
}

// (Both whole-row kernels bound a row by its 1024 thread maxima: past k =
// 512 that bound keeps too much, and larger k take the split kernel.)
constexpr int32_t kRowMaxK = kRowT / 2;

static bool use_cand_row_path(int32_t B, int32_t k, const lt_cand_t &c, int cus)
{
    if (c.block_size != 8 || c.n_blocks > 2 * kRowT || k > kRowMaxK)
        return false;
    const int force = g_force_path.load(std::memory_order_relaxed);
    if (force == 3)
        return true;
    if (force != 0)
        return false;
    return B >= 1 && (int64_t)B <= 4LL * cus;
}

// Plain rows (no candidate list) for the whole-row kernel?
static bool use_row_path(int32_t B, int32_t n_max, int32_t k)
{
    if (n_max > kRowMax || k > kRowMaxK)
        return false;
    const int force = g_force_path.load(std::memory_order_relaxed);
    if (force == 3)
        return true;
    if (force != 0)
        return false;
    return B >= 1 && n_max > kSplitT * kPlainEFine;
}

// Does a split launch with chunks of C elements fit the device in one round
// (one workgroup per compute unit) and the per-row workgroup limit?
static bool fits_one_round(int32_t B, int64_t vlen, int64_t C, int cus)
{
    const int64_t S = vlen > 0 ? (vlen + C - 1) / C : 1;
    return S <= kMaxS && (int64_t)B * S <= cus;
}

// Kernel choice. Many long rows: one streaming wave per row keeps HBM busy.
// Few rows: each row split over workgroups for latency. vlen is the virtual
// row (positions, blocks or candidate slots), C the split chunk; `streamable`
// says whether the streaming kernel handles this form at all.
static bool use_split_path(int32_t B, int64_t vlen, int64_t C, int cus, bool streamable)
{
    const int64_t S = vlen > 0 ? (vlen + C - 1) / C : 1;
    bool use_split = !streamable || S == 1 || ((int64_t)B * S <= 8LL * cus && S <= kMaxS);
    const int force = g_force_path.load(std::memory_order_relaxed);
    if (force == 1 && S <= kMaxS)
        use_split = true;
    else if (force == 2 && streamable)
        use_split = false;
    return use_split;
}

static lt_status validate_common(const float *scores, int64_t row_stride, const int32_t *lengths,
                                 int32_t B, int32_t n_max, int32_t k, const void *out)
{
    if (!scores || !lengths || !out)
        return LT_EINVAL;
    if (B < 0 || n_max < 0 || k < 1 || k > LT_K_MAX)
        return LT_EINVAL;
    if (row_stride < n_max || row_stride % 4 != 0)
        return LT_EINVAL;
    if (((uintptr_t)scores & 15u) != 0u)
        return LT_EINVAL;
    return LT_OK;
}

static lt_status check_ws(void *workspace)
{
    return ((uintptr_t)workspace & 15u) == 0u ? LT_OK : LT_EINVAL;
}

// Forms the streaming kernel does not take (the block stage with a block size
// other than 8; candidate lists with another block size, or over rows past
// kStreamShortMax) always run split, at most kMaxS workgroups per row with the
// largest chunk of their mode. Longer virtual rows are rejected on the host,
// before anything is launched.
constexpr int64_t kMaxSplitBlocks = (int64_t)kMaxS * kSplitT * kBlocksE; // 4,194,304 blocks
constexpr int64_t kMaxSplitSlots = (int64_t)kMaxS * kSplitT * kCandE;    // 8,388,608 slots
static_assert(kMaxSplitBlocks == LT_MAX_SPLIT_BLOCKS && kMaxSplitSlots == LT_MAX_SPLIT_SLOTS,
              "the header's limits follow the split chunks");
static_assert(kStreamShortMax == 536866816, "the header states the streaming row limit");

static bool blocks_supported(int32_t n_max, int32_t block_size)
{
    const int64_t nb = ((int64_t)n_max + block_size - 1) / block_size;
    return block_size == 8 || nb <= kMaxSplitBlocks;
}

static bool cand_supported(int32_t n_max, const lt_cand_t &c)
{
    const int64_t slots = (int64_t)c.n_blocks * c.block_size;
    const bool streamable = c.block_size == 8 && n_max <= kStreamShortMax;
    return streamable || slots <= kMaxSplitSlots;
}

} // namespace ltk

using namespace ltk;

extern "C" {

size_t lt_topk_workspace_bytes(int32_t B, int32_t n_max, int32_t k)
{
    (void)k;
    // A row fits one workgroup (no exchange) up to the smallest split chunk:
    // 1024 elements (the block stage with one block per thread; a block never
    // holds fewer than one position, so n_max bounds every virtual row).
    if (B <= 0 || n_max <= kSplitT * kBlocksEFine)
        return 0;
    const int64_t rows = B < kMaxSplitRows ? B : kMaxSplitRows;
    return (size_t)rows * kWsRowWords * 4u;
}

} // extern "C"

// lt_topk_run with the workspace chosen: the caller's (noalloc false) or the
// current device's built-in one.
static lt_status topk_run_impl(const float *scores, int64_t row_stride, const int32_t *lengths,
                               int32_t B, int32_t n_max, int32_t k, const lt_cand_t *cand,
                               int32_t *out_idx, void *workspace, size_t ws_bytes,
                               lt_stream_t stream, bool noalloc)
{
    lt_status st = validate_common(scores, row_stride, lengths, B, n_max, k, out_idx);
    if (st != LT_OK)
        return st;
    if (cand && (!cand->blocks || cand->n_blocks < 1 || cand->block_size < 1))
        return LT_EINVAL;
    if (cand && !cand_supported(n_max, *cand))
        return LT_EINVAL;
    if ((st = check_ws(workspace)) != LT_OK)
        return st;
    if (B == 0)
        return LT_OK;
    DeviceInfo d;
    if (device_info(d) != hipSuccess)
        return LT_EHIP;
    WsArg wa = {ws_bytes, nullptr};
    if (noalloc) {
        if (d.scratch_ptr == nullptr)
            return LT_EHIP;
        workspace = d.scratch_ptr;
        wa.bytes = kNoAllocBytes;
        wa.pending = d.scratch_pending;
    }
    KParams p = {};
    p.scores = scores;
    p.row_stride = row_stride;
    p.lengths = lengths;
    p.n_max = n_max;
    p.k = k;
    p.out = out_idx;
    p.ws = static_cast<uint32_t *>(workspace);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (cand) {
        p.cand = cand->blocks;
        p.n_cand = cand->n_blocks;
        p.bs = cand->block_size;
        const int64_t vlen = (int64_t)cand->n_blocks * cand->block_size;
        if (use_cand_row_path(B, k, *cand, d.cus))
            return launch_cand_rows(p, B, s);
        const bool streamable = cand->block_size == 8 && n_max <= kStreamShortMax;
        if (use_split_path(B, vlen, (int64_t)kSplitT * kCandE, d.cus, streamable))
            return vlen <= (int64_t)kSplitT * kCandE
                       ? launch_split<kCandE, MODE_CAND, true>(p, B, vlen, wa, s)
                   : vlen <= (int64_t)kSplitT * kCandEWhole
                       ? launch_split<kCandEWhole, MODE_CAND, true>(p, B, vlen, wa, s)
                       : launch_split<kCandE, MODE_CAND>(p, B, vlen, wa, s);
        return launch_stream<MODE_CAND>(p, B, s);
    }
    if (use_row_path(B, n_max, k))
        return launch_rows(p, B, s);
    if (use_split_path(B, n_max, (int64_t)kSplitT * kPlainE, d.cus, true))
        return fits_one_round(B, n_max, kSplitT * kPlainEFine, d.cus)
                   ? launch_split<kPlainEFine, MODE_PLAIN>(p, B, n_max, wa, s)
                   : launch_split<kPlainE, MODE_PLAIN>(p, B, n_max, wa, s);
    return launch_stream<MODE_PLAIN>(p, B, s);
}

extern "C" {

lt_status lt_topk_run(const float *scores, int64_t row_stride, const int32_t *lengths, int32_t B,
                      int32_t n_max, int32_t k, const lt_cand_t *cand, int32_t *out_idx,
                      void *workspace, size_t ws_bytes, lt_stream_t stream)
{
    return topk_run_impl(scores, row_stride, lengths, B, n_max, k, cand, out_idx, workspace,
                         ws_bytes, stream, false);
}

lt_status lt_topk_run_noalloc(const float *scores, int64_t row_stride, const int32_t *lengths,
                              int32_t B, int32_t n_max, int32_t k, const lt_cand_t *cand,
                              int32_t *out_idx, lt_stream_t stream)
{
    return topk_run_impl(scores, row_stride, lengths, B, n_max, k, cand, out_idx, nullptr, 0,
                         stream, true);
}

lt_status lt_topk_blocks(const float *scores, int64_t row_stride, const int32_t *lengths, int32_t B,
                         int32_t n_max, int32_t block_size, int32_t kb, int32_t *out_blocks,
                         void *workspace, size_t ws_bytes, lt_stream_t stream)
{
    lt_status st = validate_common(scores, row_stride, lengths, B, n_max, kb, out_blocks);
    if (st != LT_OK)
        return st;
    if (block_size < 1 || !blocks_supported(n_max, block_size))
        return LT_EINVAL;
    if ((st = check_ws(workspace)) != LT_OK)
        return st;
    if (B == 0)
        return LT_OK;
    DeviceInfo d;
    if (device_info(d) != hipSuccess)
        return LT_EHIP;
    KParams p = {};
    p.scores = scores;
    p.row_stride = row_stride;
    p.lengths = lengths;
    p.n_max = n_max;
    p.k = kb;
    p.bs = block_size;
    p.out = out_blocks;
    p.ws = static_cast<uint32_t *>(workspace);
    const int64_t vlen = ((int64_t)n_max + block_size - 1) / block_size;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const WsArg wa = {ws_bytes, nullptr};
    if (!use_split_path(B, vlen, (int64_t)kSplitT * kBlocksE, d.cus, block_size == 8))
        return launch_stream<MODE_BLOCKS>(p, B, s);
    return fits_one_round(B, vlen, kSplitT * kBlocksEFine, d.cus)
               ? launch_split<kBlocksEFine, MODE_BLOCKS>(p, B, vlen, wa, s)
               : launch_split<kBlocksE, MODE_BLOCKS>(p, B, vlen, wa, s);
}

lt_status lt_topk_two_stage(const float *scores, int64_t row_stride, const int32_t *lengths,
                            int32_t B, int32_t n_max, int32_t block_size, int32_t kb, int32_t k,
                            int32_t *out_blocks, int32_t *out_idx, void *workspace,
                            size_t ws_bytes, lt_stream_t stream)
{
    lt_status st = validate_common(scores, row_stride, lengths, B, n_max, kb, out_blocks);
    if (st != LT_OK)
        return st;
    if (!out_idx || k < 1 || k > LT_K_MAX)
        return LT_EINVAL;
    if (block_size < 1 || !blocks_supported(n_max, block_size))
        return LT_EINVAL;
    const lt_cand_t cand = {out_blocks, kb, block_size};
    if (!cand_supported(n_max, cand))
        return LT_EINVAL;
    if ((st = check_ws(workspace)) != LT_OK)
        return st;
    if (B == 0)
        return LT_OK;
    // The two calls, stream-ordered on one workspace. (Running the candidate
    // stage in the block stage's last workgroup, in one launch, measured
    // slower: compiled into the split kernel it raised the block stage's
    // registers from 87 to 126 VGPRs and its time at B = 1 from 10.7 to
    // 15.6 us, and the two stages together from 19.5 to 25.7 us.)
    st = lt_topk_blocks(scores, row_stride, lengths, B, n_max, block_size, kb, out_blocks,
                        workspace, ws_bytes, stream);
    if (st != LT_OK)
        return st;
    return lt_topk_run(scores, row_stride, lengths, B, n_max, k, &cand, out_idx, workspace,
                       ws_bytes, stream);
}

int lt_debug_force_path(int path)
{
    if (path >= 0 && path <= 3)
        return g_force_path.exchange(path);
    return g_force_path.load();
}

int lt_debug_force_fallback(int on)
{
    return g_force_fallback.exchange(on ? 1 : 0);
}

int lt_debug_force_sample(int mode)
{
    if (mode >= 0 && mode <= 2)
        return g_force_sample.exchange(mode);
    return g_force_sample.load();
}

int lt_debug_launch_shape(int32_t B, int32_t n_max, int32_t *grid_x, int32_t *grid_y,
                          int32_t *block)
{
    if (B < 1 || n_max < 0 || !grid_x || !grid_y || !block)
        return -1;
    DeviceInfo d;
    if (device_info(d) != hipSuccess)
        return -1;
    if (use_row_path(B, n_max, kRowMaxK)) {
        *grid_x = B > (1 << 30) ? (1 << 30) : B;
        *grid_y = 1;
        *block = kRowT;
        return 2;
    }
    if (use_split_path(B, n_max, (int64_t)kSplitT * kPlainE, d.cus, true)) {
        const int64_t C = fits_one_round(B, n_max, kSplitT * kPlainEFine, d.cus)
                              ? (int64_t)kSplitT * kPlainEFine
                              : (int64_t)kSplitT * kPlainE;
        const int64_t S = n_max > 0 ? ((int64_t)n_max + C - 1) / C : 1;
        *grid_x = (int32_t)S;
        *grid_y = S > 1 && B > kMaxSplitRows ? kMaxSplitRows : (B > 65535 ? 65535 : B);
        *block = kSplitT;
        return 0;
    }
    *grid_x = B;
    *grid_y = 1;
    *block = 64;
    return 1;
}

int lt_debug_empty_launch(int32_t grid_x, int32_t grid_y, int32_t block, void *stream)
{
    if (grid_x < 1 || grid_y < 1 || grid_y > 65535 || block < 1 || block > 1024)
        return -1;
    hipLaunchKernelGGL(empty_kernel, dim3(grid_x, grid_y), dim3(block), 0,
                       reinterpret_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

const char *lt_status_str(lt_status status)
{
    switch (status) {
    case LT_OK: return "LT_OK: success";
    case LT_EINVAL: return "LT_EINVAL: invalid argument (nothing launched)";
    case LT_ENOSPC: return "LT_ENOSPC: workspace too small";
    case LT_EHIP: return "LT_EHIP: HIP runtime error at launch";
    default: return "unknown lt_status";
    }
}

} // extern "C"
