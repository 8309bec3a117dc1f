// bf16 exact attention (prefill, contiguous K/V) on gfx950: the ping-pong kernel.
//
// Method (page "Donanıma Duyarlı Algoritma Tasarımı: FlashAttention"): Q, K and V are
// processed in tiles held on chip ("FlashAttention'ın Temelleri"); every query row keeps
// a running max and sum merged tile by tile ("Online Softmax Prensibi", steps 1-5) and
// the output accumulator is rescaled by the same factor, so one pass over K/V suffices;
// work is split over query rows and the next K/V tiles are fetched while the current
// ones are used ("FlashAttention-2: Optimizasyonlar ve İyileştirmeler", items 1-2). GQA:
// query head h reads K/V head h / (H / Hkv) (glossary entry "KV Cache (Anahtar-Değer
// Önbelleği)", yapayzekasozluk.tr/etiket/attention).
//
// gfx950 mapping (this design, not the pages'):
// * A SIMD issues a wave's MFMAs and its ordinary VALU work one after the other, but
//   overlaps the MFMAs of one wave with the VALU work of another. So each work-group has
//   8 waves, two per SIMD, in two groups: A = waves 0-3 (query rows 0-127 of a 256-row
//   tile), B = waves 4-7 (rows 128-255). Time is cut into slots separated by work-group
//   barriers; in every slot one group runs its matrix phase (S_j = K_j Q^T and
//   O^T += V_{j-1}^T P_{j-1}^T, 32 MFMAs per wave) while the other runs its softmax
//   phase (mask, running max, exponentials of S into P), and the groups swap each slot.
// * Per wave: 32 query rows, one per lane column, so the row max and sum are in-lane
//   reductions plus one v_permlane32_swap; scores are computed transposed
//   (v_mfma_f32_32x32x16_bf16 with K rows from LDS as A and the wave's Q in registers as
//   B) and so is the output (V^T from LDS through transposing reads as A, P^T from the
//   score registers as B).
// * K and V tiles of 64 keys go from HBM straight into LDS (buffer_load ... lds) with
//   XOR-swizzled 16-byte chunks (conflict-free operand reads), double-buffered: tile j+1
//   of K and tile j of V are loaded during period j (two slots) and published by the
//   barrier that ends it. 64 KiB of LDS, one work-group per CU.
// * The reference max used for the exponentials only moves when the row max grows by
//   more than 8 (log2 units); exponentials stay below 2^8 and the result is unchanged
//   because softmax(x) = softmax(x - c) ("FlashAttention'ın Temelleri"). The row max
//   itself is only computed when the tile's exponentials against the current reference
//   say it may have moved (a lane's share of them summing to more than 128). With a
//   window, every rise moves the reference until a wave's first tile that all its rows
//   see whole, so later tiles do not fail that check against a reference taken from a
//   few keys.
// * Causal: the work-group visits the key tiles its last row needs; a wave skips the
//   tiles entirely in its rows' future, and only tiles crossing a wave's diagonal (or
//   Nk) are masked.
// * Sliding window (glossary entry "Kayan Pencere Dikkati (Sliding Window Attention)":
//   query i at position p = Nk - Nq + i attends keys p - left .. p + right): the
//   work-group visits the band of tiles some row's window touches, a wave computes the
//   band of its own rows, and only tiles cut by a window edge (or Nk) are masked. A row's
//   first tile may hold none of its keys, so its reference max can still be -inf there.
// * Paged K/V (chunked prefill through the page table, glossary entry "KV Cache
//   (Anahtar-Değer Önbelleği)": later tokens read the stored K/V of earlier ones): a 64-key
//   tile is four 16-slot pages and each wave's direct loads cover 8 rows, half a page, so
//   a wave needs one page id per tile. Ids are read from the table (scalar loads through
//   the constant address space) a period before their tile is loaded, and each page is
//   loaded through a descriptor sized to its valid slots: slots past the sequence, pages
//   past it and out-of-range ids load as zeros and are never read. Sequences differ in
//   length, so work-groups are taken longest sequence first.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "prefill_common.h"

namespace kvfa {

namespace {
using namespace prefill;

template <int D>
struct TilePP {
    static constexpr int NW = 8;                // waves per work-group
    static constexpr int NT = 64 * NW;
    static constexpr int BM = 32 * NW;          // query rows per work-group
    static constexpr int BN = 64;               // keys per tile
    static constexpr int KB = BN / 32;          // 32-key blocks of S^T
    static constexpr int KS = D / 16;           // MFMA k-steps of Q.K
    static constexpr int DB = D / 32;           // 32-dim blocks of O^T
    static constexpr int PS = BN / 16;          // MFMA k-steps of P.V
    static constexpr int ROW = D * 2;           // bytes per K/V row
    static constexpr int TILE = BN * ROW;       // bytes of one K (or V) tile
    static constexpr int DMA = TILE / 1024 / NW;  // 1 KiB direct loads per wave per tile
    static_assert(DMA >= 1 && DMA * 1024 * NW == TILE, "whole 1 KiB loads per wave");
};

// Window sides (keys before / after the query's position); kWinUnbounded for none.
constexpr int kWinUnbounded = 1 << 29;

// The kernel's arguments, passed as one struct (so they sit at the start of the kernel
// argument segment, where the kernel reads them).
struct PPArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int H, Hkv, Nq, Nk, n_qt, BH;
    float scale_log2, tau_raw;
    int win_left, win_right;
    PagedKV pg;
};

template <int D, bool CAUSAL, bool WINDOW, bool PAGED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_pp_kernel(const PPArgs args) {
    // The arguments are loaded from the argument segment next to their first use (the
    // output pointers only at the epilogue), which keeps them out of the scalar registers
    // during the tile loop: held there, they crowd it, and the compiler then drops the
    // schedule that issues the LDS operand reads ahead of their MFMAs. (Reading them as
    // `args.x` lets the compiler load them at entry instead.) The code-object ABI places
    // the explicit arguments first in the segment, in order, so `args` is at offset 0.
    typedef const __attribute__((address_space(4))) PPArgs* ArgsPtr;
    const ArgsPtr A = (ArgsPtr)__builtin_amdgcn_kernarg_segment_ptr();
    const int n_qt = A->n_qt, BH = A->BH;
    static_assert(!(CAUSAL && WINDOW), "a causal window is the window (left, 0)");
    static_assert(!(WINDOW && PAGED), "no windowed paged variant");
    using T = TilePP<D>;
    constexpr int BN = T::BN;
    __shared__ __attribute__((aligned(1024))) char ks0[T::TILE];
    __shared__ __attribute__((aligned(1024))) char ks1[T::TILE];
    __shared__ __attribute__((aligned(1024))) char vs0[T::TILE];
    __shared__ __attribute__((aligned(1024))) char vs1[T::TILE];

    const uint16_t* __restrict__ q = A->q;
    const uint16_t* __restrict__ k = A->k;
    const uint16_t* __restrict__ v = A->v;
    const int H = A->H, Hkv = A->Hkv, Nq = A->Nq, Nk_arg = A->Nk;
    const float scale_log2 = A->scale_log2, tau_raw = A->tau_raw;
    const int win_left = A->win_left, win_right = A->win_right;
    const PagedKV pg{A->pg.page_table, A->pg.seq_lens, A->pg.max_pages, A->pg.num_pages,
                     A->pg.max_seq_len};
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
    const int grp = w >> 2;                                    // 0: group A, 1: group B
    const int col = lane & 31;  // query column of S^T / O^T owned by this lane
    const int g = lane >> 5;    // which half of the k-slots this lane supplies
    int pair, qt, b, h;
    if constexpr (PAGED) {
        // Work-groups are taken sequence by sequence, longest sequence first (ranked here
        // from seq_lens for batches of up to 64 sequences; larger batches keep their
        // order), so the short ones fill in behind the long ones.
        const int per = H * n_qt, B = BH / H;
        const int r = blockIdx.x / per;
        map_work(blockIdx.x - r * per, n_qt, H, H / Hkv, CAUSAL, h, qt);
        b = r;
        if (B <= 64) {
            __shared__ int lens_s[64];
            __shared__ int pick_s;
            if (tid < B) lens_s[tid] = pg.seq_lens[tid];
            __syncthreads();
            if (tid < B) {
                const int mine = lens_s[tid];
                int rank = 0;
                for (int o2 = 0; o2 < B; ++o2) {
                    const int other = lens_s[o2];
                    rank += (other > mine) | ((other == mine) & (o2 < tid));
                }
                if (rank == r) pick_s = tid;
            }
            __syncthreads();
            b = __builtin_amdgcn_readfirstlane(pick_s);
        }
        pair = b * H + h;
    } else {
        map_work(blockIdx.x, n_qt, BH, H / Hkv, CAUSAL || WINDOW, pair, qt);
        b = pair / H;
        h = pair % H;
    }
    const int kvh = h / (H / Hkv);
    const int q0 = qt * T::BM;
    int Nk = Nk_arg;
    if constexpr (PAGED)  // at least the Nq new tokens, at most the table's capacity
        Nk = __builtin_amdgcn_readfirstlane(min(max(pg.seq_lens[b], Nq), pg.max_seq_len));
    const int off = Nk - Nq;
    const int wrow0 = q0 + w * 32;  // first query row of this wave
    const int qrow = wrow0 + col;

    const auto rq = make_rsrc(q + (size_t)pair * Nq * D, (uint32_t)Nq * D * 2);
    const auto rk = make_rsrc(k + (PAGED ? 0 : ((size_t)b * Hkv + kvh) * Nk * D),
                              PAGED ? 0u : (uint32_t)Nk * D * 2);
    const auto rv = make_rsrc(v + (PAGED ? 0 : ((size_t)b * Hkv + kvh) * Nk * D),
                              PAGED ? 0u : (uint32_t)Nk * D * 2);

    // B operand of S^T = K Q^T: Q[qrow][16s + 8g .. +7]; rows past Nq load as zero.
    u32x4 qf[T::KS];
#pragma unroll
    for (int s = 0; s < T::KS; ++s)
        qf[s] = buf_load16(rq, (uint32_t)(qrow * D + s * 16 + g * 8) * 2);

    // Tiles j0 .. j0 + n_tiles - 1 of the work-group (every wave steps through them for
    // the barriers), tiles [jw0, jw1) this wave computes, and [jf0, jf1) the ones it can
    // take unmasked.
    const int n_all = (Nk + BN - 1) / BN;
    int j0 = 0, n_tiles = n_all, jw0 = 0, jw1 = n_all, jf0 = 0, jf1 = Nk / BN;
    const int last_row = min(q0 + T::BM, Nq) - 1;
    const int wlast = min(wrow0 + 31, Nq - 1);
    if (CAUSAL) {
        n_tiles = min(n_all, (last_row + off) / BN + 1);
        jw1 = min(n_all, (wlast + off) / BN + 1);
        jf1 = min(jf1, (wrow0 + off + 1) / BN);
    } else if (WINDOW) {
        j0 = max(0, q0 + off - win_left) / BN;
        n_tiles = min(Nk - 1, last_row + off + win_right) / BN + 1 - j0;
        jw0 = max(0, wrow0 + off - win_left) / BN;
        jw1 = min(Nk - 1, wlast + off + win_right) / BN + 1;
        // unmasked: every row's window covers the whole tile, which lies below Nk
        jf0 = max(0, wlast + off - win_left + BN - 1) / BN;
        jf1 = min(jf1, (wrow0 + off + win_right + 1) / BN);
    }
    if (wrow0 >= Nq) jw1 = jw0;  // rows past Nq: nothing to compute

    // Direct loads: the wave's i-th 1 KiB piece of a tile covers tile bytes
    // [1024 (DMA w + i), +1024); lane L fills byte 16 L of it, i.e. row r, physical chunk
    // pc, with logical chunk pc ^ swizzle(r) of row r.
    // Paged: row r of the tile is slot r % 16 of page 4j + r / 16 (a wave's rows all lie in
    // one page), rows of a page being Hkv * D elements apart.
    static_assert(T::DMA * 1024 / T::ROW == 8, "a wave loads 8 rows of a tile");
    const size_t slot_stride = (size_t)Hkv * D;
    uint32_t dk_off[T::DMA], dv_off[T::DMA];
#pragma unroll
    for (int i = 0; i < T::DMA; ++i) {
        const int byte = 1024 * (T::DMA * w + i) + 16 * lane;
        const int r = byte / T::ROW, pc = (byte % T::ROW) / 16;
        const int base = PAGED ? (int)((r % 16) * slot_stride * 2) : r * T::ROW;
        dk_off[i] = (uint32_t)(base + ((pc ^ k_swz<D>(r)) * 16));
        dv_off[i] = (uint32_t)(base + ((pc ^ v_swz<D>(r)) * 16));
    }
    // Page id of this wave's page in tile j (-1 past the sequence). The table is read
    // through the constant address space so the uniform load is a scalar one: a vector
    // load here would make its consumer wait for every tile load issued before it.
    typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
    const const_i32_ptr table_row =
        (const_i32_ptr)(pg.page_table + (PAGED ? (size_t)b * pg.max_pages : 0));
    const int wpage = w >> 1;  // this wave's page within a tile
    auto page_of = [&](int j) -> int {
        if constexpr (PAGED) {
            const int pidx = 4 * j + wpage;
            if (pidx * 16 >= Nk) return -1;
            return table_row[pidx];
        }
        return -1;
    };
    // Descriptor of the wave's page in tile j covering its valid slots (size 0 if none).
    auto page_rsrc = [&](const uint16_t* cache, int j, int pid) __attribute__((always_inline)) {
        const int valid = min(16, Nk - (4 * j + wpage) * 16);
        const bool ok = valid > 0 && (unsigned)pid < (unsigned)pg.num_pages;
        const uint16_t* base =
            cache + ((size_t)(ok ? pid : 0) * 16) * slot_stride + (size_t)kvh * D;
        return make_rsrc(base, ok ? (uint32_t)(((valid - 1) * slot_stride + D) * 2) : 0u);
    };
    // pid_cur: page of the tile whose V the current period loads; pid_nxt: of the tile
    // whose K it loads; pid_fut: read during the period for the next one.
    int pid_cur = page_of(j0), pid_nxt = page_of(j0 + 1), pid_fut = -1;
    auto load_k = [&](int j, char* dst, int pid) __attribute__((always_inline)) {
        if constexpr (PAGED) {
            const auto r = page_rsrc(k, j, pid);
#pragma unroll
            for (int i = 0; i < T::DMA; ++i)
                buf_load16_lds(r, dst + 1024 * (T::DMA * w + i), dk_off[i], 0u);
        } else {
#pragma unroll
            for (int i = 0; i < T::DMA; ++i)
                buf_load16_lds(rk, dst + 1024 * (T::DMA * w + i), dk_off[i],
                               (uint32_t)(j * T::TILE));
        }
    };
    auto load_v = [&](int j, char* dst, int pid) __attribute__((always_inline)) {
        if constexpr (PAGED) {
            const auto r = page_rsrc(v, j, pid);
#pragma unroll
            for (int i = 0; i < T::DMA; ++i)
                buf_load16_lds(r, dst + 1024 * (T::DMA * w + i), dv_off[i], 0u);
        } else {
#pragma unroll
            for (int i = 0; i < T::DMA; ++i)
                buf_load16_lds(rv, dst + 1024 * (T::DMA * w + i), dv_off[i],
                               (uint32_t)(j * T::TILE));
        }
    };

    // Per-lane LDS read offsets. K operand (kb, s): row 32 kb + col, logical chunk 2s + g.
    // V^T operand (t, db, half): rows 16t + 8 half + 4(G/2) + e, logical chunk
    // 4 db + 2(G%2) + a/2, byte 8(a%2) in it (G = lane/16, lane%16 = a + 4e).
    int kr_off[T::KS];
#pragma unroll
    for (int s = 0; s < T::KS; ++s)
        kr_off[s] = col * T::ROW + (((2 * s + g) ^ k_swz<D>(col)) * 16);
    const int vG = lane >> 4, va = lane & 3, ve = (lane >> 2) & 3;
    const int vrow = (vG >> 1) * 4 + ve;
    int vr_off[T::DB];
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
        vr_off[db] = vrow * T::ROW + (((4 * db + 2 * (vG & 1) + (va >> 1)) ^ v_swz<D>(vrow)) * 16) +
                     8 * (va & 1);

    float m_used = -INFINITY;  // raw-score reference max of this lane's query
    float l_part = 0.f;        // this lane's share of the row sum
    f32x16 oacc[T::DB];
#pragma unroll
    for (int i = 0; i < T::DB; ++i) oacc[i] = f32x16{};
    f32x16 sacc[T::KB];  // S^T of the tile between its matrix and softmax phases
    u32x4 pf[T::PS];     // P^T (bf16) of the tile between its softmax and matrix phases

    // Matrix phase: S_j = K_j Q^T (if qk) and O^T += V_{j-1}^T P_{j-1}^T (if pv).
    auto matrix_phase = [&](const char* kst, const char* vst, bool qk, bool pv)
                            __attribute__((always_inline)) {
        if (qk) {
#pragma unroll
            for (int kb = 0; kb < T::KB; ++kb) {
                sacc[kb] = f32x16{};
#pragma unroll
                for (int s = 0; s < T::KS; ++s) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(kst + kr_off[s] + kb * 32 * T::ROW);
                    sacc[kb] = mfma32x32x16(a, qf[s], sacc[kb]);
                }
            }
            // Each K operand read goes three MFMAs ahead of its use.
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // DS reads
#pragma unroll
            for (int i = 0; i < T::KB * T::KS - 3; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
        }
        if (pv) {
#pragma unroll
            for (int t = 0; t < T::PS; ++t)
#pragma unroll
                for (int db = 0; db < T::DB; ++db) {
                    // keys 16t + 4g + {0..3} and 16t + 8 + 4g + {0..3} at dim 32db + col
                    const u32x2 a0 = lds_read_tr(vst + vr_off[db] + (t * 16) * T::ROW);
                    const u32x2 a1 = lds_read_tr(vst + vr_off[db] + (t * 16 + 8) * T::ROW);
                    const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
                    oacc[db] = mfma32x32x16(a, pf[t], oacc[db]);
                }
            // The V^T operand reads go two MFMAs ahead of their use.
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < T::PS * T::DB - 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
    };

    // Softmax phase of tile j: mask, running max (lazy reference), P = exp2 into pf.
    auto softmax_phase = [&](const int j) __attribute__((always_inline)) {
        // No fusing of a separate multiply and add into one FMA here (the compiler may do it
        // or not depending on the code around): the row sum's rescale-then-add must round
        // the same way in the single-pass kernel and the statistics pass.
#pragma clang fp contract(off)
        if (j < jf0 || j >= jf1) {
            // key offset inside the tile of element (kb, i) is kb*32 + 8*(i/4) + 4g + i%4;
            // it is dead past the row's last key and past Nk (and, for a window, before
            // the row's first key).
            int lim = Nk - 1 - j * BN - 4 * g;
            if (CAUSAL) lim = min(lim, qrow + off - j * BN - 4 * g);
            if (WINDOW) {
                lim = min(lim, qrow + off + win_right - j * BN - 4 * g);
                const int lo = qrow + off - win_left - j * BN - 4 * g;
#pragma unroll
                for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kb * 32 + (i >> 2) * 8 + (i & 3);
                        if (key > lim || key < lo) sacc[kb][i] = -INFINITY;
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (kb * 32 + (i >> 2) * 8 + (i & 3) > lim) sacc[kb][i] = -INFINITY;
            }
        }
        // Fast path: the exponentials against the current reference, without the row max.
        // If this lane's share of the row sum grew by at most 128, none of them exceeds
        // ~128 (the sum's rounding hides less than 128 while it stays below 2^26), so no
        // score lies more than 8 (log2 units) above the reference: the path below would
        // keep the reference and compute the same values, and the tile is done. Otherwise
        // (or while the reference is still -inf) the wave takes that path.
        // With a window, a row's first visited tiles may hold only a few of its keys, and the
        // low reference they give (a move needs a rise of more than 8) would fail the check
        // on most later tiles. So until the wave's first tile that every one of its rows sees
        // whole (jf0), and at it, any rise moves the reference (the -inf start moves anyway),
        // and only after it may a tile take the fast path. A window unbounded on the left has
        // jf0 = 0, where every reference is still -inf: it computes exactly what the causal
        // kernel does.
        const bool settled = !WINDOW || j > jf0;
        if (settled) {
            const float mb0 = m_used * scale_log2;
            float l_new = l_part;
#pragma unroll
            for (int t = 0; t < T::PS; ++t) {
                const int kb = t >> 1, base = (t & 1) * 8;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float p0 = fast_exp2(fmaf(sacc[kb][base + 2 * u], scale_log2, -mb0));
                    const float p1 = fast_exp2(fmaf(sacc[kb][base + 2 * u + 1], scale_log2, -mb0));
                    pf[t][u] = pack_bf16x2(p0, p1);
                    l_new += p0 + p1;
                }
            }
            const bool ok = m_used != -INFINITY && l_new <= l_part + 128.f;
            if (!__builtin_amdgcn_ballot_w64(!ok)) {
                l_part = l_new;
                return;
            }
        }
        // Without a window every row attends key 0, so after its first tile the max is
        // finite; with one the reference stays -inf until the row's first key, and a row
        // that does not move keeps alpha = 1 (never -inf - -inf).
        float mx = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        mx = fmaxf(mx, xor32(mx));
        const float m_cand = fmaxf(m_used, mx);
        const bool move = m_cand > m_used + (settled ? tau_raw : 0.f);
        if (__builtin_amdgcn_ballot_w64(move)) {
            // Only rows whose max moved change their reference (alpha = 1 elsewhere), so
            // a row's arithmetic never depends on the other rows of the wave.
            const float m_new = move ? m_cand : m_used;
            const float alpha = move ? fast_exp2((m_used - m_new) * scale_log2) : 1.f;
            m_used = m_new;
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < T::DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        }
        const float mb = (WINDOW && m_used == -INFINITY) ? 0.f : m_used * scale_log2;
#pragma unroll
        for (int t = 0; t < T::PS; ++t) {
            const int kb = t >> 1, base = (t & 1) * 8;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float p0 = fast_exp2(fmaf(sacc[kb][base + 2 * u], scale_log2, -mb));
                const float p1 = fast_exp2(fmaf(sacc[kb][base + 2 * u + 1], scale_log2, -mb));
                pf[t][u] = pack_bf16x2(p0, p1);
                l_part += p0 + p1;  // fp32 sum of the unrounded exponentials
            }
        }
    };

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // Period p = slots 2p and 2p+1 works on tile j = j0 + p; K_j is in stage p&1,
    // V_{j-1} in stage (p-1)&1.
    //   slot 2j:   A: matrix phase (QK_j, PV_{j-1})   B: softmax of tile j-1
    //   slot 2j+1: B: matrix phase (QK_j, PV_{j-1})   A: softmax of tile j
    // K_{j+1} and V_j are loaded at the start of the period; the barrier that ends it
    // (after each wave's own loads complete) publishes them. The barrier between the two
    // slots waits for nothing but the other group. Each group runs its own copy of the
    // loop (the same number of barriers), straight-line code for one role.
    auto period = [&](const int p, auto par, auto role) __attribute__((always_inline)) {
        const int j = j0 + p;
        constexpr int pv = decltype(par)::value;
        constexpr bool is_a = decltype(role)::value == 0;
        const char* k_cur = pv ? ks1 : ks0;   // K_j
        char* k_nxt = pv ? ks0 : ks1;         // receives K_{j+1}
        const char* v_prev = pv ? vs0 : vs1;  // V_{j-1}
        char* v_cur = pv ? vs1 : vs0;         // receives V_j
        if (p + 1 < n_tiles) load_k(j + 1, k_nxt, pid_nxt);
        if (p < n_tiles) load_v(j, v_cur, pid_cur);
        if constexpr (PAGED) pid_fut = page_of(j + 2);
        const bool qk = j >= jw0 && j < jw1, pvv = p >= 1 && j - 1 >= jw0 && j - 1 < jw1;
        if constexpr (is_a) {
            matrix_phase(k_cur, v_prev, qk, pvv);
            __builtin_amdgcn_s_barrier();
            if (qk) softmax_phase(j);
        } else {
            if (pvv) softmax_phase(j - 1);
            __builtin_amdgcn_s_barrier();
            matrix_phase(k_cur, v_prev, qk, pvv);
        }
        __syncthreads();
        if constexpr (PAGED) {
            pid_cur = pid_nxt;
            pid_nxt = pid_fut;
        }
    };
    auto run = [&](auto role) __attribute__((always_inline)) {
        int p = 0;
        for (; p + 1 <= n_tiles; p += 2) {
            period(p, P0{}, role);
            period(p + 1, P1{}, role);
        }
        if (p <= n_tiles) period(p, P0{}, role);  // periods 0 .. n_tiles
    };

    load_k(j0, ks0, pid_cur);
    __syncthreads();
    if (grp == 0) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});

    // ---- epilogue: O = O_acc / l, lse = M + ln L ----
    // A lane holds 8-byte pieces of its row spread over the row, so the wave first writes
    // its 32 rows to LDS (the tile stages are free now: every wave has passed the last
    // period's barrier, and that period loads nothing) and then stores whole rows, each
    // instruction four full rows of HBM (16-byte chunks XOR-swizzled by row in LDS).
    const float l = l_part + xor32(l_part);
    const float inv = 1.f / l;
    constexpr int CH = T::ROW / 16;  // 16-byte chunks per row
    static_assert(2 * 32 * T::ROW == T::TILE, "two waves' rows fill one stage");
    char* ost = (w >> 1) == 0 ? ks0 : (w >> 1) == 1 ? ks1 : (w >> 1) == 2 ? vs0 : vs1;
    ost += (w & 1) * 32 * T::ROW;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // dims 32 db + 8 r + 4 g .. +3: logical chunk 4 db + r, byte 8 g in it
            const u32x2 pk = {pack_bf16x2(oacc[db][r * 4 + 0] * inv, oacc[db][r * 4 + 1] * inv),
                              pack_bf16x2(oacc[db][r * 4 + 2] * inv, oacc[db][r * 4 + 3] * inv)};
            *reinterpret_cast<u32x2*>(ost + col * T::ROW + (((4 * db + r) ^ (col % CH)) * 16) +
                                      8 * g) = pk;
        }
    uint16_t* const o = A->o;
    float* const lse = A->lse;
    uint16_t* obase = o + ((size_t)pair * Nq + wrow0) * D;
#pragma unroll
    for (int i = 0; i < 32 * T::ROW / 1024; ++i) {
        const int byte = 1024 * i + 16 * lane;
        const int row = byte / T::ROW, pc = (byte % T::ROW) / 16;
        const u32x4 val = *reinterpret_cast<const u32x4*>(ost + byte);
        if (wrow0 + row < Nq)
            *reinterpret_cast<u32x4*>(obase + row * D + ((pc ^ (row % CH)) * 8)) = val;
    }
    if (lse != nullptr && g == 0 && qrow < Nq)
        lse[(size_t)pair * Nq + qrow] = (m_used * scale_log2 + fast_log2(l)) * kLn2;
}

template <int D, bool CAUSAL, bool WINDOW, bool PAGED = false>
hipError_t launch_pp(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int Hkv, int Nq, int Nk, float scale, hipStream_t stream,
                     int win_left = kWinUnbounded, int win_right = kWinUnbounded,
                     PagedKV pg = PagedKV{nullptr, nullptr, 0, 0, 0}) {
    using T = TilePP<D>;
    const int n_qt = (Nq + T::BM - 1) / T::BM;
    const int BH = B * H;
    const float scale_log2 = scale * kLog2e;
    const float tau_raw = 8.0f / scale_log2;  // move the reference max past +8 in log2 units
    const PPArgs args{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                      static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse,
                      H, Hkv, Nq, Nk, n_qt, BH, scale_log2, tau_raw, win_left, win_right, pg};
    hipLaunchKernelGGL((fwd_pp_kernel<D, CAUSAL, WINDOW, PAGED>), dim3(n_qt * BH),
                       dim3(T::NT), 0, stream, args);
    return hipGetLastError();
}

}  // namespace

// Work decomposition by launch size. The ping-pong kernel's 256-row work-groups each sweep
// their rows' whole key range; with few of them the launch lasts as long as one sweep while
// most compute units idle. The key-split kernel (64-row work-groups whose key range runs in
// four parts side by side) shortens that chain 4x but reads every K/V tile once per 64 rows
// instead of once per 256. Measured (MI355X, us, ping-pong -> key-split): at 64 ping-pong
// work-groups B2 H8 N1024 d64 causal 20.3 -> 9.8, B1 H8 N2048 d128 causal 43.4 -> 22.7; at
// 128 B1 H8 N4096 d128 causal 81.2 -> 49.5, B1 H32 Hkv8 N1024 d128 25.8 -> 20.1, B4 H8
// N1024 d128 25.7 -> 24.4; at 256 (before the key-split kernel shared its Q tiles) B2 H16
// N2048 d64 37.5 -> 39.1. The key-split kernel takes
// launches of up to 128 ping-pong work-groups (half the compute units) whose key range is
// longer than two 64-key tiles; with at most 128 keys there is no chain to split, and its
// barrier and larger work-groups cost ~1 us (B2 H8 N128 d64 causal: 5.9 -> 6.3 us).
constexpr int kComputeUnits = 256;

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                           hipStream_t stream) {
    const long long pp_groups = (long long)((Nq + TilePP<128>::BM - 1) / TilePP<128>::BM) * B * H;
    if (pp_groups <= kComputeUnits / 2 && Nk > 128)
        return launch_fwd_bf16_key_split(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal, scale,
                                         stream);
    if (d == 128)
        return causal
                   ? launch_pp<128, true, false>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream)
                   : launch_pp<128, false, false>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream);
    return causal ? launch_pp<64, true, false>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream)
                  : launch_pp<64, false, false>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream);
}

hipError_t launch_fwd_bf16_window(const void* q, const void* k, const void* v, void* o,
                                  float* lse, int B, int H, int Hkv, int Nq, int Nk, int d,
                                  int window_left, int window_right, float scale,
                                  hipStream_t stream) {
    const int left = window_left < 0 ? kWinUnbounded : window_left;
    const int right = window_right < 0 ? kWinUnbounded : window_right;
    if (d == 128)
        return launch_pp<128, false, true>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream,
                                           left, right);
    return launch_pp<64, false, true>(q, k, v, o, lse, B, H, Hkv, Nq, Nk, scale, stream, left,
                                      right);
}

hipError_t launch_fwd_bf16_paged(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* page_table, const int32_t* seq_lens, void* o,
                                 float* lse, int B, int H, int Hkv, int Nq, int d, int num_pages,
                                 int max_pages_per_seq, int max_seq_len, int causal, float scale,
                                 hipStream_t stream) {
    const PagedKV pg{page_table, seq_lens, max_pages_per_seq, num_pages, max_seq_len};
    constexpr int U = kWinUnbounded;
    if (d == 128)
        return causal ? launch_pp<128, true, false, true>(q, k_cache, v_cache, o, lse, B, H, Hkv,
                                                          Nq, max_seq_len, scale, stream, U, U, pg)
                      : launch_pp<128, false, false, true>(q, k_cache, v_cache, o, lse, B, H,
                                                           Hkv, Nq, max_seq_len, scale, stream,
                                                           U, U, pg);
    return causal ? launch_pp<64, true, false, true>(q, k_cache, v_cache, o, lse, B, H, Hkv, Nq,
                                                     max_seq_len, scale, stream, U, U, pg)
                  : launch_pp<64, false, false, true>(q, k_cache, v_cache, o, lse, B, H, Hkv, Nq,
                                                      max_seq_len, scale, stream, U, U, pg);
}

}  // namespace kvfa
