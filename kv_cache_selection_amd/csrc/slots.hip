// slots.hip -- slot leases for the KV pools (host side) and the two device
// operations they need: moving a token's rows to another slot, and checking
// page-table entries against slot generations.
//
// The article's memory-ledger section makes requests finishable, cancellable
// and safe to follow with new requests through leases, generation markers
// and a tail ring buffer, after which the cache capacity and slots return to
// their initial values. Here:
//   - a pool of n physical slots, each with a generation counter; free slots
//     are handed out lowest first;
//   - a lease (one request) may take a tail ring of R slots when it opens:
//     token t goes to ring slot ring[t % R]; when token t >= R arrives, token
//     t - R leaves the ring for a body slot taken from the pool (its rows are
//     moved ring -> body before the new token overwrites the ring slot);
//     without a ring every token takes a body slot;
//   - closing a lease returns all its slots and increments their generations,
//     so page-table entries recorded under an older generation are stale.
#include "libqsa.h"
#include "qsa_internal.h"

#include <map>
#include <mutex>
#include <set>
#include <vector>

struct qsa_slot_pool {
    std::mutex mu;
    int64_t n = 0;
    std::vector<uint32_t> gen;
    std::set<int32_t> free;                 // ordered: lowest first
    struct Lease {
        std::vector<int32_t> ring, body;
        int64_t t = 0;
    };
    std::map<int32_t, Lease> leases;
    int32_t next_id = 1;

    bool take(int32_t *s)
    {
        if (free.empty())
            return false;
        *s = *free.begin();
        free.erase(free.begin());
        return true;
    }
    void give(int32_t s)
    {
        gen[s]++;
        free.insert(s);
    }
};

extern "C" {

qsa_status_t qsa_pool_create(int64_t n_slots, qsa_slot_pool_t **pool)
{
    if (!pool || n_slots < 1 || n_slots > INT32_MAX)
        return QSA_ERR_INVALID_ARGUMENT;
    qsa_slot_pool *p = new (std::nothrow) qsa_slot_pool;
    if (!p)
        return QSA_ERR_OUT_OF_SLOTS;
    p->n = n_slots;
    p->gen.assign((size_t)n_slots, 0u);
    for (int64_t s = 0; s < n_slots; s++)
        p->free.insert(p->free.end(), (int32_t)s);
    *pool = p;
    return QSA_OK;
}

void qsa_pool_destroy(qsa_slot_pool_t *pool)
{
    delete pool;
}

qsa_status_t qsa_pool_open(qsa_slot_pool_t *pool, int32_t ring_slots, int32_t *lease)
{
    if (!pool || !lease || ring_slots < 0)
        return QSA_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> g(pool->mu);
    if ((int64_t)ring_slots > (int64_t)pool->free.size())
        return QSA_ERR_OUT_OF_SLOTS;
    qsa_slot_pool::Lease L;
    for (int32_t i = 0; i < ring_slots; i++) {
        int32_t s;
        pool->take(&s);
        L.ring.push_back(s);
    }
    const int32_t id = pool->next_id++;
    pool->leases.emplace(id, std::move(L));
    *lease = id;
    return QSA_OK;
}

qsa_status_t qsa_pool_next(qsa_slot_pool_t *pool, int32_t lease, qsa_slot_plan_t *plan)
{
    if (!pool || !plan)
        return QSA_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> g(pool->mu);
    auto it = pool->leases.find(lease);
    if (it == pool->leases.end())
        return QSA_ERR_INVALID_ARGUMENT;
    qsa_slot_pool::Lease &L = it->second;
    const int64_t t = L.t;
    const int64_t R = (int64_t)L.ring.size();
    qsa_slot_plan_t p;
    p.token = t;
    p.spill_token = -1;
    p.spill_from = p.spill_to = -1;
    p.spill_generation = 0;
    if (R == 0) {
        int32_t s;
        if (!pool->take(&s))
            return QSA_ERR_OUT_OF_SLOTS;
        L.body.push_back(s);
        p.slot = s;
    } else {
        p.slot = L.ring[(size_t)(t % R)];
        if (t >= R) {
            int32_t to;
            if (!pool->take(&to))
                return QSA_ERR_OUT_OF_SLOTS;
            L.body.push_back(to);
            p.spill_token = t - R;
            p.spill_from = p.slot;
            p.spill_to = to;
            p.spill_generation = pool->gen[(size_t)to];
        }
    }
    p.generation = pool->gen[(size_t)p.slot];
    L.t++;
    *plan = p;
    return QSA_OK;
}

qsa_status_t qsa_pool_close(qsa_slot_pool_t *pool, int32_t lease)
{
    if (!pool)
        return QSA_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> g(pool->mu);
    auto it = pool->leases.find(lease);
    if (it == pool->leases.end())
        return QSA_ERR_INVALID_ARGUMENT;
    for (int32_t s : it->second.ring)
        pool->give(s);
    for (int32_t s : it->second.body)
        pool->give(s);
    pool->leases.erase(it);
    return QSA_OK;
}

int64_t qsa_pool_free_slots(qsa_slot_pool_t *pool)
{
    if (!pool)
        return -1;
    std::lock_guard<std::mutex> g(pool->mu);
    return (int64_t)pool->free.size();
}

qsa_status_t qsa_pool_generations(qsa_slot_pool_t *pool, uint32_t *gen_out)
{
    if (!pool || !gen_out)
        return QSA_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> g(pool->mu);
    for (int64_t s = 0; s < pool->n; s++)
        gen_out[s] = pool->gen[(size_t)s];
    return QSA_OK;
}

} // extern "C"

namespace qsa {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// One wave per sequence: token[b] (or -1) moves from its current slot to
// to_slot[b] in every layer's pool; the page table and, when given, the
// token-generation table follow.
__global__ __launch_bounds__(64) void move_kernel(AppendLayers ly, int n_layers, const int64_t *__restrict__ token,
                                                  const int32_t *__restrict__ to_slot,
                                                  const uint32_t *__restrict__ to_gen, int32_t *__restrict__ pt,
                                                  int64_t pt_stride, int64_t n_slots, uint32_t *__restrict__ tok_gen)
{
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int64_t t = token[b];
    const int32_t to = to_slot[b];
    if (t < 0 || t >= pt_stride || to < 0 || (int64_t)to >= n_slots)
        return;
    const int32_t from = pt[(int64_t)b * pt_stride + t];
    if (from < 0 || (int64_t)from >= n_slots)
        return;
    for (int l = 0; l < n_layers; l++) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(ly.pool[l] + (int64_t)from * kRowBytes);
        u32x4 *dst = reinterpret_cast<u32x4 *>(ly.pool[l] + (int64_t)to * kRowBytes);
        const u32x4 a = src[lane], c = src[lane + 64];
        dst[lane] = a;
        dst[lane + 64] = c;
    }
    if (lane == 0) {
        pt[(int64_t)b * pt_stride + t] = to;
        if (tok_gen)
            tok_gen[(int64_t)b * pt_stride + t] = to_gen ? to_gen[b] : 0u;
    }
}

// stale[b] += number of tokens t < ctx_len[b] in this workgroup's chunk whose
// slot's generation differs from the one recorded when the token was placed
// (or whose slot is out of range). Grid (chunks of kCheckChunk tokens, B);
// stale[] is cleared first, and a chunk adds to it only when it found
// something, so a clean cache costs no atomics.
constexpr int kCheckThreads = 256;
constexpr int kCheckChunk = 8192;

__global__ __launch_bounds__(kCheckThreads) void check_gen_kernel(const int32_t *__restrict__ ctx_len,
                                                                  int64_t pt_stride, const int32_t *__restrict__ pt,
                                                                  const uint32_t *__restrict__ tok_gen,
                                                                  const uint32_t *__restrict__ slot_gen,
                                                                  int64_t n_slots, int32_t *__restrict__ stale)
{
    __shared__ uint32_t red[kCheckThreads / 64];
    const int b = blockIdx.y;
    int64_t L = ctx_len[b];
    L = L < 0 ? 0 : (L > pt_stride ? pt_stride : L);
    const int64_t t0 = (int64_t)blockIdx.x * kCheckChunk;
    if (t0 >= L)
        return;
    const int64_t t1 = t0 + kCheckChunk < L ? t0 + kCheckChunk : L;
    uint32_t bad = 0;
    for (int64_t t = t0 + threadIdx.x; t < t1; t += kCheckThreads) {
        const int32_t s = pt[(int64_t)b * pt_stride + t];
        const bool ok = s >= 0 && (int64_t)s < n_slots && slot_gen[s] == tok_gen[(int64_t)b * pt_stride + t];
        bad += ok ? 0u : 1u;
    }
    for (int o = 32; o >= 1; o >>= 1)
        bad += __shfl_xor(bad, o);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = bad;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t tot = 0;
        for (int w = 0; w < kCheckThreads / 64; w++)
            tot += red[w];
        if (tot)
            atomicAdd(&stale[b], (int32_t)tot);
    }
}

} // namespace

hipError_t launch_move(const AppendLayers &ly, int n_layers, int batch, const int64_t *token, const int32_t *to_slot,
                       const uint32_t *to_gen, int32_t *pt, int64_t pt_stride, int64_t n_slots, uint32_t *tok_gen,
                       hipStream_t s)
{
    hipLaunchKernelGGL(move_kernel, dim3((unsigned)batch), dim3(64), 0, s, ly, n_layers, token, to_slot, to_gen, pt,
                       pt_stride, n_slots, tok_gen);
    return hipGetLastError();
}

hipError_t launch_check_gen(const int32_t *ctx_len, int batch, int64_t pt_stride, const int32_t *pt,
                            const uint32_t *tok_gen, const uint32_t *slot_gen, int64_t n_slots, int32_t *stale,
                            hipStream_t s)
{
    hipError_t e = launch_fill_i32(stale, batch, 0, s);
    if (e != hipSuccess)
        return e;
    dim3 grid((unsigned)((pt_stride + kCheckChunk - 1) / kCheckChunk), (unsigned)batch);
    hipLaunchKernelGGL(check_gen_kernel, grid, dim3(kCheckThreads), 0, s, ctx_len, pt_stride, pt, tok_gen, slot_gen,
                       n_slots, stale);
    return hipGetLastError();
}

} // namespace qsa
