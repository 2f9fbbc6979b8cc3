// KV cache addressing shared by the cache writer (RoPE kernel) and the
// attention kernels.  A request's cache is either contiguous or paged.
//
//   contiguous: per (layer, KV head) a key block [capacity][dh] followed (in
//     the [layer][K / V][head] order) by a transposed value block
//     [dh][capacity]: kv + ((layer * 2 + kind) * hkv + head) * capacity * dh.
//   paged: 64-token pages taken from a pool; token t of the request lives in
//     page pt[t / 64] at slot t % 64.  A page holds every layer and head of its
//     64 tokens, [layer][K / V][head][64 * dh]: keys [64][dh], transposed
//     values [dh][64]; pages are page_elems elements apart from the pool base.
//
// Either way a 64-token block of one (layer, head) is 64 key rows of dh
// contiguous elements plus dh value rows of 64 consecutive tokens (row stride
// vstride), which is the attention kernel's tile.
#pragma once
#include "common.h"
#include "kernels.h"

namespace dlm {

template <typename T>
struct KVBlock {
    T* k;            // key of the block's token i: k + i * dh
    T* vt;           // value dimension d of token i: vt + d * vstride + i
    long vstride;
};

template <typename T>
__device__ __forceinline__ KVBlock<T> kv_block(const SeqTab& s, int sq, int layer, int hkv, int head, int dh,
                                               int blk) {
    KVBlock<T> b;
    T* base = (T*)s.kv[sq];
    if (s.pt[sq]) {
        T* pg = base + (long)s.pt[sq][blk] * s.page_elems;
        b.k = pg + ((long)(layer * 2 + 0) * hkv + head) * KV_PAGE * dh;
        b.vt = pg + ((long)(layer * 2 + 1) * hkv + head) * KV_PAGE * dh;
        b.vstride = KV_PAGE;
    } else {
        const long cap = s.cap[sq];
        b.k = base + ((long)(layer * 2 + 0) * hkv + head) * cap * dh + (long)blk * KV_PAGE * dh;
        b.vt = base + ((long)(layer * 2 + 1) * hkv + head) * cap * dh + (long)blk * KV_PAGE;
        b.vstride = cap;
    }
    return b;
}

}  // namespace dlm
