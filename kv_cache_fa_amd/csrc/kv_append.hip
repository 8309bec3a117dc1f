// Writing new tokens' keys and values into the paged KV cache.
//
// Method: glossary entry "KV Cache (Anahtar-Değer Önbelleği)" (yapayzekasozluk.tr, tag
// "Attention") and the "KV Önbelleği" topic of "SGLang'de Flash Attention Arka Ucu:
// Temeller ve KV Önbelleği Uygulaması": the K/V computed for a token are stored once and
// read by every later step instead of being recomputed. This library keeps them in fixed
// pages: per layer, K and V are [num_pages][16 slots][Hkv][d] bf16, sequence s owns the
// pages listed in its row of the page table, and its token at position p sits in slot
// p % 16 of page page_table[s][p / 16]. Appending the K/V of n_new tokens that start at
// position start_pos[s] is then a pure scatter: each 16-byte chunk of a token's [Hkv][d]
// row is copied to its slot. One thread moves one chunk of K and the same chunk of V, so
// the kernel streams 2 x (read + write) x num_seqs x n_new x Hkv x d x 2 bytes.
#include "common.h"
#include "launch.h"

namespace kvfa {
namespace {

// Index arithmetic in Idx (32-bit when the chunk count allows: 64-bit division is a long
// instruction sequence on the GPU). The new rows are loaded before the page-table lookup so
// the two memory round trips overlap.
template <typename Idx>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ start_pos, long long n_chunks_ll, int chunks_per_tok, int n_new,
    int num_pages, int max_pages) {
    const Idx n_chunks = (Idx)n_chunks_ll;
    const Idx stride = (Idx)gridDim.x * blockDim.x;
    for (Idx c = (Idx)blockIdx.x * blockDim.x + threadIdx.x; c < n_chunks; c += stride) {
        const u32x4 kx = k_new[c], vx = v_new[c];
        const Idx tok = c / (Idx)chunks_per_tok;  // s * n_new + t
        const int within = (int)(c - tok * (Idx)chunks_per_tok);
        const int s = (int)(tok / (Idx)n_new), t = (int)(tok - (Idx)s * n_new);
        const long long pos = (long long)start_pos[s] + t;
        if (pos < 0 || pos >= (long long)max_pages * 16) continue;  // outside the table: dropped
        const int pid = page_table[(size_t)s * max_pages + (int)(pos >> 4)];
        if ((unsigned)pid >= (unsigned)num_pages) continue;  // unassigned page: dropped
        const size_t dst = ((size_t)pid * 16 + (size_t)(pos & 15)) * chunks_per_tok + within;
        k_cache[dst] = kx;
        v_cache[dst] = vx;
    }
}

}  // namespace

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* page_table, const int32_t* start_pos, int num_seqs,
                            int n_new, int Hkv, int d, int num_pages, int max_pages_per_seq,
                            hipStream_t stream) {
    const int chunks_per_tok = Hkv * d / 8;
    const long long n_chunks = (long long)num_seqs * n_new * chunks_per_tok;
    // Enough work-groups to cover the chip several times over; the loop strides the rest.
    const long long want = (n_chunks + 255) / 256;
    const int grid = (int)(want < 8192 ? want : 8192);
    if (n_chunks + (long long)grid * 256 < (1ll << 31))
        hipLaunchKernelGGL(kv_append_kernel<int>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const u32x4*>(k_new), static_cast<const u32x4*>(v_new),
                           static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache),
                           page_table, start_pos, n_chunks, chunks_per_tok, n_new, num_pages,
                           max_pages_per_seq);
    else
        hipLaunchKernelGGL(kv_append_kernel<long long>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const u32x4*>(k_new), static_cast<const u32x4*>(v_new),
                           static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache),
                           page_table, start_pos, n_chunks, chunks_per_tok, n_new, num_pages,
                           max_pages_per_seq);
    return hipGetLastError();
}

}  // namespace kvfa
