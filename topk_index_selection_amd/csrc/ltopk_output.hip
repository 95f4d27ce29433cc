// Output variants of a selection for its consumer, CSA's sparse attention over
// the selected compressed positions (AICon 2026 Shenzhen speaker page,
// aicon.infoq.cn: abstract and outline 一.1). The pages give no layout for what
// the consumer receives; these calls reorder a row's selected indices
// (ascending, or in selection order), return the scores at them, and gather
// the selected rows of a compressed-KV cache. See include/ltopk.h.
//
// gfx950 (wave64) only.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ltopk.h"

namespace lto {

// Order-preserving map from fp32 bits to an unsigned key, the one the
// selection ranks by: larger key = higher score, -0.0 shares +0.0's key,
// every NaN gets 1 (below -inf's 0x007FFFFF).
__device__ __forceinline__ uint32_t order_key(uint32_t u)
{
    uint32_t key = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
    key = u == 0x80000000u ? 0x80000000u : key;
    key = (u & 0x7fffffffu) > 0x7f800000u ? 1u : key;
    return key;
}

struct OrderParams {
    const float *scores;
    int64_t row_stride;
    int32_t n_max;
    int32_t k;
    int32_t order;
    int32_t row0;
    int32_t *idx;
    float *vals;
};

constexpr int kOrderT = 256;

// One workgroup per row. Each slot becomes a 64-bit sort key whose low half
// is the index: ascending order sorts the index itself; selection order sorts
// ~(key(score) << 32 | ~index), i.e. higher score first and lower index first
// on equal scores. Empty slots (and indices outside [0, n_max)) become ~0 and
// sort last, coming out as -1. A bitonic sort over N >= k keys in LDS; the
// write-back also fills the values (the score at the index, -inf if empty).
//
// The scores sit at random positions of their rows, so each one read costs a
// whole cache line from HBM. In selection order with values, where the score
// is needed twice, it is read once: its bits stay in LDS by slot, and the low
// half of the sort key carries the slot below the index's bits (index order
// is unchanged, as indices are distinct) whenever both fit 32 bits.
template <int N>
__global__ __launch_bounds__(kOrderT) void order_kernel(OrderParams p)
{
    __shared__ uint64_t key[N];
    __shared__ uint32_t raw[N];
    constexpr int LOGN = __builtin_ctz(N);
    const int64_t row = (int64_t)p.row0 + blockIdx.x;
    int32_t *ir = p.idx + row * p.k;
    const float *sr = p.scores + row * p.row_stride;
    const int tid = threadIdx.x;
    // index bits of n_max; the slot rides below them if they leave room
    const int ib = p.n_max <= 1 ? 0 : 32 - __builtin_clz((uint32_t)(p.n_max - 1));
    const bool carry = p.order == LT_ORDER_RANK && p.vals != nullptr && ib + LOGN <= 32;
    const uint32_t imask = ib >= 32 ? 0xffffffffu : ((1u << ib) - 1u);

    if (p.order == LT_ORDER_ASIS) {
        for (int j = tid; j < p.k; j += kOrderT) {
            const int32_t i = ir[j];
            p.vals[row * p.k + j] = (i >= 0 && i < p.n_max) ? sr[i] : -__builtin_inff();
        }
        return;
    }
    for (int j = tid; j < N; j += kOrderT) {
        uint64_t kk = ~0ull;
        if (j < p.k) {
            const int32_t i = ir[j];
            if (i >= 0 && i < p.n_max) {
                if (p.order == LT_ORDER_RANK) {
                    const uint32_t bits = __float_as_uint(sr[i]);
                    const uint32_t sk = order_key(bits);
                    // (imask - i) falls as i rises, like ~i
                    const uint32_t lo = carry ? (((imask - (uint32_t)i) << LOGN) | (uint32_t)j)
                                              : (uint32_t)~(uint32_t)i;
                    raw[j] = bits;
                    kk = ~(((uint64_t)sk << 32) | lo);
                } else {
                    kk = (uint32_t)i;
                }
            }
        }
        key[j] = kk;
    }
    __syncthreads();
    for (int size = 2; size <= N; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < N / 2; t += kOrderT) {
                const int lo = 2 * t - (t & (stride - 1));
                const int hi = lo + stride;
                const uint64_t a = key[lo], c = key[hi];
                if ((a > c) == ((lo & size) == 0)) {
                    key[lo] = c;
                    key[hi] = a;
                }
            }
            __syncthreads();
        }
    }
    for (int j = tid; j < p.k; j += kOrderT) {
        const uint64_t kk = key[j];
        if (carry) {
            const uint32_t lo = ~(uint32_t)kk; // (imask - i) << LOGN | slot
            const bool full = kk != ~0ull;
            const int32_t i = full ? (int32_t)(imask - (lo >> LOGN)) : -1;
            ir[j] = i;
            p.vals[row * p.k + j] = full ? __uint_as_float(raw[lo & (N - 1)]) : -__builtin_inff();
            continue;
        }
        const int32_t i = kk == ~0ull ? -1 : (int32_t)(uint32_t)kk;
        ir[j] = i;
        if (p.vals)
            p.vals[row * p.k + j] = i >= 0 ? sr[i] : -__builtin_inff();
    }
}

struct GatherParams {
    const uint8_t *kv;
    int64_t kv_stride;
    int64_t kv_batch_stride;
    int64_t n_kv;
    const int32_t *idx;
    uint8_t *out;
    int32_t k;
    uint32_t chunks;   // 16-byte chunks per row
    int32_t row0;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGatherT = 256;
constexpr int kGatherU = 4; // chunks per thread, loads issued together

// out[b, j] = kv[b][idx[b, j]] (row_bytes each), zeros for empty slots. The
// (slot, chunk) pairs of a row are numbered t = j * chunks + c, so a
// workgroup's stores are one contiguous span of the output and its loads are
// whole cache rows. Grid: (ceil(k * chunks / (256 * 4)), rows).
__global__ __launch_bounds__(kGatherT) void gather_kernel(GatherParams p)
{
    const int64_t b = (int64_t)p.row0 + blockIdx.y;
    const uint32_t total = (uint32_t)p.k * p.chunks;
    const uint32_t t0 = blockIdx.x * (uint32_t)(kGatherT * kGatherU) + threadIdx.x;
    const int32_t *ir = p.idx + b * p.k;
    const uint8_t *kvb = p.kv + b * p.kv_batch_stride;
    u32x4 *ob = reinterpret_cast<u32x4 *>(p.out) + b * (int64_t)total;
    u32x4 v[kGatherU];
#pragma unroll
    for (int u = 0; u < kGatherU; ++u) {
        const uint32_t t = t0 + (uint32_t)(u * kGatherT);
        v[u] = u32x4{0u, 0u, 0u, 0u};
        if (t < total) {
            const uint32_t j = t / p.chunks;
            const uint32_t c = t - j * p.chunks;
            const int32_t i = ir[j];
            if (i >= 0 && (int64_t)i < p.n_kv)
                v[u] = *reinterpret_cast<const u32x4 *>(kvb + (int64_t)i * p.kv_stride +
                                                         (int64_t)c * 16);
        }
    }
#pragma unroll
    for (int u = 0; u < kGatherU; ++u) {
        const uint32_t t = t0 + (uint32_t)(u * kGatherT);
        if (t < total)
            __builtin_nontemporal_store(v[u], ob + t);
    }
}

template <int N>
static void launch_order(const OrderParams &q, int32_t rows, hipStream_t s)
{
    hipLaunchKernelGGL(order_kernel<N>, dim3(rows), dim3(kOrderT), 0, s, q);
}

} // namespace lto

using namespace lto;

extern "C" {

lt_status lt_topk_order(const float *scores, int64_t row_stride, int32_t B, int32_t n_max,
                        int32_t k, int32_t order, int32_t *idx, float *out_vals,
                        lt_stream_t stream)
{
    if (!idx || B < 0 || n_max < 0 || k < 1 || k > LT_K_MAX)
        return LT_EINVAL;
    if (order != LT_ORDER_ASIS && order != LT_ORDER_INDEX && order != LT_ORDER_RANK)
        return LT_EINVAL;
    const bool need_scores = order == LT_ORDER_RANK || out_vals != nullptr;
    if (need_scores && (!scores || row_stride < n_max))
        return LT_EINVAL;
    if (B == 0 || (order == LT_ORDER_ASIS && !out_vals))
        return LT_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    OrderParams q = {};
    q.scores = scores;
    q.row_stride = row_stride;
    q.n_max = n_max;
    q.k = k;
    q.order = order;
    q.idx = idx;
    q.vals = out_vals;
    for (int64_t r0 = 0; r0 < B; r0 += 1 << 30) {
        q.row0 = (int32_t)r0;
        const int32_t rows = (int32_t)(B - r0 < (1 << 30) ? B - r0 : (1 << 30));
        if (k <= 128)
            launch_order<128>(q, rows, s);
        else if (k <= 512)
            launch_order<512>(q, rows, s);
        else if (k <= 2048)
            launch_order<2048>(q, rows, s);
        else
            launch_order<4096>(q, rows, s);
    }
    return hipGetLastError() == hipSuccess ? LT_OK : LT_EHIP;
}

lt_status lt_gather_rows(const void *kv, int64_t kv_stride, int64_t kv_batch_stride, int64_t n_kv,
                         int32_t row_bytes, const int32_t *idx, int32_t B, int32_t k, void *out,
                         lt_stream_t stream)
{
    if (!kv || !idx || !out || B < 0 || k < 1 || k > LT_K_MAX || n_kv < 0)
        return LT_EINVAL;
    if (row_bytes < 16 || row_bytes > (1 << 20) || row_bytes % 16 != 0)
        return LT_EINVAL;
    if (kv_stride < row_bytes || kv_stride % 16 != 0 || kv_batch_stride < 0 ||
        kv_batch_stride % 16 != 0)
        return LT_EINVAL;
    if (reinterpret_cast<uintptr_t>(kv) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
        return LT_EINVAL;
    if (B == 0)
        return LT_OK;
    GatherParams q = {};
    q.kv = static_cast<const uint8_t *>(kv);
    q.kv_stride = kv_stride;
    q.kv_batch_stride = kv_batch_stride;
    q.n_kv = n_kv;
    q.idx = idx;
    q.out = static_cast<uint8_t *>(out);
    q.k = k;
    q.chunks = (uint32_t)(row_bytes / 16);
    const uint32_t total = (uint32_t)k * q.chunks;
    const uint32_t per_wg = (uint32_t)(kGatherT * kGatherU);
    const uint32_t gx = (total + per_wg - 1) / per_wg;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int32_t r0 = 0; r0 < B; r0 += 65535) {
        q.row0 = r0;
        const int32_t rows = B - r0 < 65535 ? B - r0 : 65535;
        hipLaunchKernelGGL(gather_kernel, dim3(gx, rows), dim3(kGatherT), 0, s, q);
    }
    return hipGetLastError() == hipSuccess ? LT_OK : LT_EHIP;
}

} // extern "C"
