// Shared pieces of the bf16 prefill kernels (prefill_bf16.hip, prefill_pp.hip): the LDS
// swizzles of K and V tiles, the work-group -> (batch*head, q tile) order and the
// transposing LDS read. gfx950 only.
#pragma once

#include "common.h"

namespace kvfa {
namespace prefill {

// XOR swizzles of the 16-byte chunks of a tile row (a direct-to-LDS load writes 1 KiB
// contiguously, so rows cannot be padded). K: the 16 rows read together by a 16-lane
// group for one MFMA operand land on 16 different bank groups. V: the 4 rows gathered by
// one transposing read land on 4 different 64-byte bank groups.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
    if constexpr (D == 128) return row & 15;
    else return (row >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
    if constexpr (D == 128) return 4 * (row & 3);
    else return 4 * ((row >> 1) & 1);
}

// Swizzle for a tile read both ways: as rows (16 consecutive rows, one chunk) and through
// transposing reads (4 consecutive rows, an aligned group of 4 chunks). For D = 128 the
// row's low two bits pick the group of 4 chunks and bits 2-3 the chunk inside it, so 16
// consecutive rows hit 16 different chunks and 4 consecutive rows 4 different groups.
// For D = 64 two rows share a 256-byte bank cycle, so the same holds per row parity.
template <int D>
__device__ __forceinline__ int kt_swz(int row) {
    if constexpr (D == 128) return 4 * (row & 3) + ((row >> 2) & 3);
    else return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}

// Work-group id -> (batch*H + head, q tile). The dispatcher places work-group i on XCD
// i % 8, and each XCD has its own L2. When the (batch, head) count is a multiple of 8,
// XCD x owns a contiguous block of (batch, head) pairs; if that block holds whole GQA
// groups (the g query heads that read one K/V head), the XCD finishes one group's q
// tiles before starting the next, so its L2 only has to hold one K/V head at a time.
// Within that order causal q tiles run longest first.
__device__ __forceinline__ void map_work(int id, int n_qt, int BH, int g, bool causal,
                                         int& pair, int& qt) {
    int r;
    if ((BH & 7) == 0) {
        const int per = BH >> 3, slot = id >> 3, x = id & 7;
        if (per % g == 0) {
            const int span = g * n_qt;              // work-groups of one GQA group
            const int grp = slot / span, rem = slot % span;
            pair = x * per + grp * g + rem % g;
            r = rem / g;
        } else {
            pair = x * per + slot % per;
            r = slot / per;
        }
    } else {
        pair = id % BH;
        r = id / BH;
    }
    qt = causal ? n_qt - 1 - r : r;
}

// Paged K/V: K and V live in a paged cache [page][16 slots][Hkv][D] and sequence b's
// token t sits in slot t % 16 of page page_table[b][t / 16]. The keys of sequence b are
// its seq_lens[b] cached tokens (at least the Nq new ones, at most max_seq_len); its Nq
// queries are the last Nq of them.
struct PagedKV {
    const int32_t* page_table;  // [B, max_pages]
    const int32_t* seq_lens;    // [B]
    int max_pages, num_pages, max_seq_len;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16). Within each 16-lane group, source lane
// a + 4e points at 4 consecutive bf16 of row e (e = 0..3), column block a; lane i of
// the group receives column i of rows 0..3.
__device__ __forceinline__ u32x2 lds_read_tr(const char* p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) char*)p);
    return __builtin_bit_cast(u32x2, v);
}

}  // namespace prefill
}  // namespace kvfa
