// Feature-sharded embedding lookup, EmbeddingWithReplicateOutput ("Module 并行：
// 实现 DP/TP/CP/PP 组合", section "DP / TP / CP / PP 并行实现", "Tensor
// Parallel": the weight is Shard(1) on embedding_dim, the token ids are
// Replicate, and the output is all-gathered back to Replicate).
//
// With all P shards on one GPU the lookup and the all-gather are one pass:
// shard i copies row ids[t] of its [V, D/P] table into row t of the output at
// feature offset i*D/P (or into its own [T, D/P] block, the Shard(-1) output
// before the all-gather).  Pure data movement, HBM-bound: each (token, shard)
// row piece is read once and written once.
//
// One wavefront per token and group of up to 8 shards: the id is read once
// (a scalar load), the group's shard pointers are fetched before any data, and
// the group's pieces are loaded into registers 1 KB per instruction (16 bytes
// per lane) before any is stored, so eight independent HBM reads per
// wavefront are in flight at once; loads and stores are non-temporal, since
// every byte is touched once.  For the Llama-8B table (4096 tokens x 8 shards
// of 1 KB at random rows of 128 MB shard tables, a new batch of ids every
// launch) this takes 12.8-12.9 us (5.2 TB/s), and 12.6 us over one [V, D]
// table; the platform's torch.nn.functional.embedding over that one table
// takes 12.9 us, the per-shard gathers followed by torch.cat 46 us.  Measured
// alternatives (same box, graph-replayed): one wavefront per (token, shard)
// piece 15.1 us (one chain of id load, data load and store per 1 KB), 2 or 4
// shards per wavefront 14.0 us, two tokens per wavefront 16.0 us, cached
// loads 13.5 us.  An id outside [0, V) gives zero pieces and sets the caller's
// flag.
#include "kernels.h"

#include <type_traits>

namespace tpl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int EMB_THREADS = 256;

constexpr int EMB_GROUP = 8;   // shards per wavefront

__global__ __launch_bounds__(EMB_THREADS)
void embedding_vec(EmbedArgs e, int es) {
    const int64_t w = (int64_t)blockIdx.x * (EMB_THREADS / 64) +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t groups = (e.P + EMB_GROUP - 1) / EMB_GROUP;
    if (w >= e.T * groups) return;
    const int64_t t = w / groups;
    const int i0 = (int)(w - t * groups) * EMB_GROUP;
    const int64_t id = e.ids[t];
    const int64_t bytes = e.Ds * es;
    const bool bad = id < 0 || id >= e.V;
    if (bad && e.bad && lane == 0) *e.bad = 1;
    const char *src[EMB_GROUP];
    char *dst[EMB_GROUP];
#pragma unroll
    for (int k = 0; k < EMB_GROUP; ++k) {
        const int i = min(i0 + k, e.P - 1);
        src[k] = (const char *)e.e_shard[i] + (bad ? 0 : id) * e.lde * es;
        dst[k] = (char *)e.Y + ((int64_t)i * e.y_shard + t * e.ldy) * es;
    }
    // 1 KB chunks of each piece (one for D/P <= 512 bf16 features)
    for (int64_t o = (int64_t)lane * 16; o - lane * 16 < bytes; o += 1024) {
        u32x4 v[EMB_GROUP];
#pragma unroll
        for (int k = 0; k < EMB_GROUP; ++k) {
            v[k] = u32x4{0u, 0u, 0u, 0u};
            if (i0 + k < e.P && o < bytes && !bad)
                v[k] = __builtin_nontemporal_load((const u32x4 *)(src[k] + o));
        }
#pragma unroll
        for (int k = 0; k < EMB_GROUP; ++k)
            if (i0 + k < e.P && o < bytes) __builtin_nontemporal_store(v[k], (u32x4 *)(dst[k] + o));
    }
}

// Any alignment: one thread per output element.
template <int ES>
__global__ __launch_bounds__(EMB_THREADS)
void embedding_scalar(EmbedArgs e) {
    const int64_t idx = (int64_t)blockIdx.x * EMB_THREADS + threadIdx.x;
    const int64_t per_t = (int64_t)e.P * e.Ds;
    if (idx >= e.T * per_t) return;
    const int64_t t = idx / per_t;
    const int64_t rem = idx - t * per_t;
    const int i = (int)(rem / e.Ds);
    const int64_t c = rem - (int64_t)i * e.Ds;
    const int64_t id = e.ids[t];
    typedef typename std::conditional<ES == 2, uint16_t, uint32_t>::type T;
    T *y = (T *)e.Y + (int64_t)i * e.y_shard + t * e.ldy + c;
    if (id < 0 || id >= e.V) {
        *y = 0;
        if (e.bad && c == 0) *e.bad = 1;
        return;
    }
    *y = ((const T *)e.e_shard[i])[id * e.lde + c];
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

hipError_t launch_embedding(const EmbedArgs &e, int es, hipStream_t s) {
    if (e.T == 0 || e.Ds == 0) return hipSuccess;
    bool vec = (e.Ds * es) % 16 == 0 && (e.lde * es) % 16 == 0 && (e.ldy * es) % 16 == 0 &&
               (e.y_shard * es) % 16 == 0 && aligned16(e.Y);
    for (int i = 0; i < e.P && vec; ++i) vec = aligned16(e.e_shard[i]);
    if (vec) {
        const int64_t waves = e.T * ((e.P + EMB_GROUP - 1) / EMB_GROUP);
        const int64_t blocks = (waves + EMB_THREADS / 64 - 1) / (EMB_THREADS / 64);
        if (blocks > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
        embedding_vec<<<dim3((unsigned)blocks), dim3(EMB_THREADS), 0, s>>>(e, es);
    } else {
        const int64_t blocks = (e.T * e.P * e.Ds + EMB_THREADS - 1) / EMB_THREADS;
        if (blocks > 0x7FFFFFFFll) return hipErrorInvalidConfiguration;
        if (es == 2) embedding_scalar<2><<<dim3((unsigned)blocks), dim3(EMB_THREADS), 0, s>>>(e);
        else embedding_scalar<4><<<dim3((unsigned)blocks), dim3(EMB_THREADS), 0, s>>>(e);
    }
    return hipGetLastError();
}

}  // namespace tpl
