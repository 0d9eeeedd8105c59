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
// One wavefront per (token, shard) piece, consecutive wavefronts taking the
// shards of one token in order, so the pieces of an output row are written
// by neighbouring wavefronts.  Each lane moves 16 bytes per pass (one 1 KB
// run per wavefront instruction); loads and stores are non-temporal, since
// every byte is touched once.  For 4096 tokens x 8 shards of 1 KB at random
// rows of 128 MB tables this takes ~15 us per launch (4.4 TB/s), the rate of
// random 1 KB reads from HBM: two, four or eight pieces per wavefront (all
// loads before the stores) ran 16.2, 20.3 and 47.4 us, 64- or 1024-thread
// workgroups the same as 256.  An id outside [0, V) gives a zero piece and
// sets the caller's flag.
#include "kernels.h"

#include <type_traits>

namespace tpl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int EMB_THREADS = 256;

__global__ __launch_bounds__(EMB_THREADS)
void embedding_vec(EmbedArgs e, int es) {
    const int64_t w = ((int64_t)blockIdx.x * EMB_THREADS + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (w >= e.T * e.P) return;
    const int64_t t = w / e.P;
    const int i = (int)(w - t * e.P);
    const int64_t id = e.ids[t];
    char *y = (char *)e.Y + ((int64_t)i * e.y_shard + t * e.ldy) * es;
    const int64_t bytes = e.Ds * es;
    if (id < 0 || id >= e.V) {
        for (int64_t o = (int64_t)lane * 16; o < bytes; o += 1024)
            *(u32x4 *)(y + o) = u32x4{0u, 0u, 0u, 0u};
        if (e.bad && lane == 0) *e.bad = 1;
        return;
    }
    const char *src = (const char *)e.e_shard[i] + id * e.lde * es;
    for (int64_t o = (int64_t)lane * 16; o < bytes; o += 1024) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4 *)(src + o));
        __builtin_nontemporal_store(v, (u32x4 *)(y + o));
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
        const int64_t blocks = (e.T * e.P * 64 + EMB_THREADS - 1) / EMB_THREADS;
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
