// Single-token decode against a paged KV cache: split-K attention + log-sum-exp merge.
//
// Method: glossary entry "KV Cache (Anahtar-Değer Önbelleği)" (yapayzekasozluk.tr,
// tag "Attention"): the new token's query reads the cached K/V of every earlier token
// (its own K/V already appended); the cache lives in fixed-size pages; under GQA
// several query heads share one K/V head. The softmax over the cached keys uses the
// running max / running sum merge of page "Donanıma Duyarlı Algoritma Tasarımı:
// FlashAttention", "Online Softmax Prensibi" steps 1-5, both inside a segment (page by
// page) and across segments (the combine kernel merges (O_k, lse_k) pairs, the same
// algebra expressed through one log-sum-exp per part).
//
// gfx950 mapping (this design):
// * Work-groups per (KV head, head group): the cached pages of all sequences, laid end to
//   end, are cut into equal ranges of R pages (R from the total, read in-kernel from
//   seq_lens), one range per work-group, so every work-group reads the same amount and
//   all of them end together (with one work-group per fixed-size split, the launch ended
//   with a few long splits running on an otherwise idle chip: a work-group's read rate is
//   bound by its loads in flight, not shared out). A range may span several sequences; each
//   piece of a sequence inside it is a segment with its own partial result. 4 waves; wave w
//   takes pages w, w+4, ... of a segment. All query heads of the GQA group are served from
//   one read of each K/V page, so every cached byte is read once.
// * Scores: S^T[token][head] = K_page Q^T with v_mfma_f32_16x16x32_bf16 — one page
//   (16 tokens) is exactly the MFMA's 16 rows, the group's heads fill its columns.
//   The MFMA wants one token per lane of a 16-lane group, HBM wants whole rows per
//   16 lanes: K pages therefore go HBM -> LDS by direct loads (buffer_load ... lds, each
//   instruction 1 KiB of whole rows, 16-byte chunks XOR-swizzled by row) into a
//   per-wave double buffer, and the A operand is read from there without bank
//   conflicts.
// * P.V, bf16 cache with one KV head per work-group: O^T[dim][head] += V^T P^T on
//   v_mfma_f32_16x16x16_bf16. The score accumulator of S^T already holds P^T in the B
//   operand's layout (lane: head column n, tokens 4 kq .. 4 kq + 3), so the probabilities
//   never leave the lane; V pages go HBM -> LDS like K (second per-wave double buffer)
//   and come back as the A operand through transposing reads (ds_read_b64_tr_b16). The
//   accumulator is 4 fp32 per 16 dims per lane whatever the head count (a 16-head group
//   held 128 per lane on FMAs, one wave per SIMD).
// * The same on an e4m3 cache with d = 128 (unless its KV heads are read in pairs): the V rows
//   come through registers (as below), are converted exactly to bf16 and written into the
//   bf16 stage right before their P.V.
// * P.V otherwise (KV head pairs; groups of up to 4 heads over 32 or more sequences; an
//   e4m3 cache with d = 64): on the VALU. A lane owns one 16-byte chunk
//   of V rows (8 dims) for a subset of the page's tokens and accumulates all heads of the
//   group; the probabilities reach it through a small per-wave LDS table. The lane takes
//   its tokens two at a time: each dim's two values and the two probabilities (rounded to
//   bf16, as the matrix-unit paths round them) form bf16 pairs, and one v_dot2c_f32_bf16
//   adds both products to the fp32 accumulator (half the instructions of fp32 FMAs). With
//   KV head pairs (256-element rows) one score lane produces both tokens of a pair, so the
//   table holds the probabilities already paired.
// * A segment's partial result (normalised O_k, lse_k in log2 units) goes to the
//   caller's workspace, slot k = its work-group's index among those covering the
//   sequence; a second kernel merges a sequence's slots in order.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "prefill_common.h"

namespace kvfa {

namespace {

constexpr int kPage = 16;
constexpr int kWaves = 4;
// A wave keeps the ids of its pages of a segment in its 64 lanes, plus the two it
// prefetches past the last one: at most 62 pages per wave and segment.
constexpr int kMaxRangePages = kWaves * 62;
// Range plan: a work-group reads at least rmin pages (so a sequence has at most
// ceil(pages / rmin) + 1 segments: the workspace's slots per head) and at most
// kMaxRangePages, so at least min_wgs work-groups per (KV head, head group) are launched
// for the longest possible cache. The kernel uses its target count (set at launch from the
// resident work-groups), or more when the actual pages need them.
struct DecodePlan {
    int rmin, max_slots, min_wgs;
};
DecodePlan decode_plan(int num_seqs, int max_seq_len) {
    const long long max_pages = (max_seq_len + kPage - 1) / kPage;
    const long long bound = (long long)num_seqs * max_pages;  // pages over all sequences
    DecodePlan p;
    p.rmin = (int)std::min<long long>(kMaxRangePages, std::max<long long>(4, (max_pages + 31) / 32));
    p.max_slots = (int)((max_pages + p.rmin - 1) / p.rmin) + 1;
    p.min_wgs = (int)std::min<long long>((bound + kMaxRangePages - 1) / kMaxRangePages, 1LL << 30);
    return p;
}

// FP8 = true: the cache holds e4m3 bytes with one scale per KV head for K and one for V
// (dequantised value = byte value x scale). K bytes are converted exactly to bf16 for the
// score MFMA and V bytes exactly to bf16 for the P.V (v_dot2c pairs or the matrix unit's
// stage); the K scale is folded into the softmax scale and the V scale is applied to each
// partial result, so the arithmetic is that of the dequantised cache. Each cached token costs half the bytes of the bf16 cache.
// PAIR: a work-group serves two neighbouring KV heads, GH / 2 query columns each, and reads
// their rows as one row of twice the length (two rows of one token are adjacent in the
// page): HBM serves longer contiguous pieces faster (128 -> 256 bytes for e4m3 with d = 128
// or bf16 with d = 64, 256 -> 512 bytes for bf16 with d = 128). Q is zero outside its own
// head's half of the row, so one score product covers both heads.
// Per-KV-head scale arrays exist only for an e4m3 cache: the bf16 instantiations take
// nullptr_t in their place, so no code path of theirs can read through one.
template <bool FP8>
using ScalePtr = std::conditional_t<FP8, const float*, std::nullptr_t>;

template <int D, int GH, bool FP8, bool PAIR = false, bool MMA = false>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ kcache,
    const void* __restrict__ vcache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, float* __restrict__ o_part,
    float* __restrict__ lse_part, int* __restrict__ n_slots, const int* __restrict__ plan,
    int num_seqs, int H, int Hkv,
    int g, int n_hg, int num_pages, int max_pages, int max_seq_len, int rmin, int max_slots,
    int wg_target, float scale_log2_in, ScalePtr<FP8> k_scale, ScalePtr<FP8> v_scale) {
    constexpr int ES = FP8 ? 1 : 2;    // bytes per cached element
    using KVec = std::conditional_t<FP8, u32x2, u32x4>;  // 8 cached elements
    constexpr int NK = PAIR ? 2 : 1;   // KV heads per work-group
    constexpr int DR = NK * D;         // elements of one row read (token, NK KV heads)
    constexpr int G2 = GH / NK;        // query columns per KV head
    static_assert(!PAIR || (GH == 8 && (D * ES == 128 || D * ES == 256)),
                  "pairs: 128- or 256-byte rows, four query columns per KV head");
    constexpr int CH = DR / 8;         // 8-element chunks per row read
    constexpr int TG = 64 / CH;        // token groups of the P.V lane layout
    constexpr int TPL = kPage / TG;    // tokens per lane in P.V
    constexpr int KS = DR / 32;        // MFMA k-steps over the row
    constexpr int ROWB = DR * ES;      // bytes of one row read
    constexpr int KCH = ROWB / 16;     // 16-byte chunks per row
    constexpr int PAGEB = kPage * ROWB;            // bytes of one page's K rows
    constexpr int KDMA = PAGEB / 1024;             // 1 KiB direct loads per page
    static_assert(KDMA >= 1 && KDMA * 1024 == PAGEB, "whole 1 KiB loads per page");
    constexpr bool MPV = MMA;                      // P.V on the matrix unit
    // KV head pairs with 256-element rows (two token groups): P.V by v_dot2c_f32_bf16, two
    // tokens of one dim per instruction (the lane's tokens tg + 2i come in pairs 4 ip + tg,
    // 4 ip + tg + 2, both held by one score lane).
    constexpr bool DOT = PAIR && TG == 2;
    static_assert(!DOT || TPL == 8, "dot2 P.V: eight tokens per lane");
    // The other VALU P.V layouts pair the lane's tokens tg + TG (2 ip) and tg + TG (2 ip + 1),
    // which different score lanes produce: the probabilities stay fp32 in LDS and the P.V
    // lane packs each pair itself.
    static_assert(MPV || TPL % 2 == 0, "dot2 P.V: an even number of tokens per lane");
    static_assert(!MMA || !PAIR, "matrix-unit P.V: one KV head");
    static_assert(!MMA || !FP8 || D == 128, "matrix-unit P.V on an e4m3 cache: d = 128");
    constexpr int VB = D / 16;                     // 16-dim blocks of O^T (MPV)
    // MPV: the V stage holds bf16 rows. A bf16 cache's pages go there by direct loads; an
    // e4m3 cache's V rows come through registers (as for the VALU P.V) and are converted
    // into the stage just before their P.V.
    constexpr int VROWB = MPV ? D * 2 : ROWB;      // bytes of one V stage row
    constexpr int VPAGEB = kPage * VROWB;          // bytes of one V stage
    constexpr bool VDMA = MPV && !FP8;             // V by direct loads into the stage
    // Per wave: two K stages (separate arrays, so the compiler can tell a read of one from
    // the direct loads into the other); after the wave's loop its partial output for the
    // cross-wave merge reuses the first stage when it fits.
    __shared__ __attribute__((aligned(1024))) char kst_a[kWaves][PAGEB];
    __shared__ __attribute__((aligned(1024))) char kst_b[kWaves][PAGEB];
    // V stages of the matrix-unit P.V (bf16 rows).
    __shared__ __attribute__((aligned(1024))) char vst_a[kWaves][MPV ? VPAGEB : 16];
    __shared__ __attribute__((aligned(1024))) char vst_b[kWaves][MPV ? VPAGEB : 16];
    // The waves' partial outputs [GH][D] for the cross-wave merge: in the first K stage
    // when they fit, with MPV in both K stages or (e4m3, whose K stages are the smaller
    // ones) both V stages (rows of heads [0, HPS) in the first), else in an array of their
    // own.
    constexpr bool RO_IN_A = GH * D * 4 <= PAGEB;
    constexpr bool RO_IN_AB = MPV && !RO_IN_A;
    constexpr int RO_STAGE = FP8 ? VPAGEB : PAGEB;  // bytes of each stage the merge uses
    static_assert(!RO_IN_AB || GH * D * 4 <= 2 * RO_STAGE, "two stages hold the partial output");
    __shared__ float red_o_x[RO_IN_A || RO_IN_AB ? 1 : kWaves * GH * D];
    auto red_o_row = [&](int ww, int hh) -> float* {  // head hh's D floats of wave ww
        if constexpr (RO_IN_A) {
            return reinterpret_cast<float*>(kst_a[ww]) + hh * D;
        } else if constexpr (RO_IN_AB) {
            constexpr int HPS = RO_STAGE / (D * 4);
            char* const first = FP8 ? vst_a[ww] : kst_a[ww];
            char* const second = FP8 ? vst_b[ww] : kst_b[ww];
            return reinterpret_cast<float*>(hh < HPS ? first : second) + (hh % HPS) * D;
        } else {
            return red_o_x + (ww * GH + hh) * D;
        }
    };
    __shared__ float p_lds[kWaves][MPV || DOT ? 1 : kPage][MPV || DOT ? 1 : GH];  // fp32 P
    // DOT: the probabilities of tokens (4 q + r, 4 q + r + 2), r = 0, 1, as bf16 pairs.
    __shared__ __attribute__((aligned(16))) uint32_t p2_lds[kWaves][DOT ? kPage / 2 : 1][DOT ? GH : 1];
    __shared__ float a_lds[kWaves][GH];
    __shared__ float red_m[kWaves][GH];
    __shared__ float red_l[kWaves][GH];

    const int kvh = NK * (blockIdx.x / n_hg), hg = blockIdx.x % n_hg;  // (first) KV head
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
    const int n = lane & 15;     // head column of S^T held by this lane
    const int kq = lane >> 4;    // k-slot group / token quad of S^T
    const int tg = lane / CH, c = lane % CH;  // P.V layout: token group, V chunk
    const int h0 = kvh * g + hg * GH;
    const int nheads = min(GH, g - hg * GH);
    // Column n's KV head (of the NK) and query head, and whether that head exists. The
    // MFMA has 16 columns; columns n >= GH are padding: they take the last KV head of the
    // work-group (so every per-head array they index stays in range) and are never
    // valid, so their Q stays zero and nothing of theirs is stored.
    const int kn = PAIR ? min(n / G2, NK - 1) : 0, hn = PAIR ? n % G2 : n;
    const int head_n = PAIR ? (kvh + kn) * g + hn : h0 + n;
    const bool col_ok = PAIR ? (n < GH && hn < g) : n < nheads;
    const size_t tok_stride = (size_t)Hkv * D;  // elements between consecutive slots
    // Softmax scale in log2 units (times the K scale for an fp8 cache) and the V scale.
    float scale_log2 = scale_log2_in, v_sc = 1.f;
    if constexpr (FP8) {
        scale_log2 *= k_scale[kvh + kn];  // per column: the column's KV head
        v_sc = v_scale[kvh];              // (pairs take theirs per column in the merge)
    }
    // Move the reference max past +8 in log2 units (with a zero K scale every score is 0:
    // the first page then moves the reference and every later one keeps it).
    const float tau_raw = scale_log2 > 0.f ? 8.0f / scale_log2 : 0.f;

    // Issue the loads of the wave's it-th page (K rows as the MFMA A operand, V chunks for
    // the P.V lanes). Returns false for an out-of-range page id, which is never read.
    // Loads are issued unconditionally (a zero-size descriptor for an invalid page id
    // makes them return zeros without touching memory), so the wait counts stay exact.
    // The cache is read once per call: the loads carry the nontemporal hint.
    const uint32_t span = (uint32_t)((kPage - 1) * tok_stride + DR) * ES;
    const uint32_t v_off = (uint32_t)(tg * tok_stride + c * 8) * ES;
    // K direct loads: lane L of the i-th 1 KiB piece fills stage byte 1024 i + 16 L, i.e.
    // row r, physical chunk pc, with logical chunk pc ^ (r % KCH) of cached row r.
    uint32_t kd_off[KDMA];
#pragma unroll
    for (int i = 0; i < KDMA; ++i) {
        const int byte = 1024 * i + 16 * lane;
        const int r = byte / ROWB, pc = (byte % ROWB) / 16;
        kd_off[i] = (uint32_t)(r * tok_stride * ES + ((pc ^ (r % KCH)) * 16));
    }
    // A operand of k-step j: token n, elements 32 j + 8 kq .. +7 (8 ES bytes).
    int kr_off[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const int b = (32 * j + 8 * kq) * ES;
        kr_off[j] = n * ROWB + (((b / 16) ^ (n % KCH)) * 16) + b % 16;
    }
    // MPV: V stage rows are tokens of VROWB bytes, 16-byte chunks XOR-swizzled by row so that
    // a transposing read (16-lane group kq: tokens 4 kq + e, e = 0..3, 8 bytes of dims
    // 16 vb + 4 a each) and its neighbour group (tokens 4 kq + 4 + e), which the LDS serves
    // together, hit 32 different bank pairs.
    auto v_swz_dec = [](int r) -> int {
        if constexpr (VROWB == 256) return 4 * (r & 3) + 2 * ((r >> 2) & 1);
        else return 2 * ((r >> 1) & 3);
    };
    static_assert(!MPV || VROWB == 256 || VROWB == 128, "MPV: d = 128 or 64");
    uint32_t vd_off[VDMA ? KDMA : 1];
    int vr_off[MPV ? VB : 1];
    if constexpr (MPV) {
        if constexpr (VDMA) {
#pragma unroll
            for (int i = 0; i < KDMA; ++i) {
                const int byte = 1024 * i + 16 * lane;
                const int r = byte / VROWB, pc = (byte % VROWB) / 16;
                vd_off[i] = (uint32_t)(r * tok_stride * ES + ((pc ^ v_swz_dec(r)) * 16));
            }
        }
        // Source lane a + 4 e of group kq points at token 4 kq + e, dims 16 vb + 4 a .. +3:
        // logical chunk 2 vb + a / 2, byte 8 (a % 2) in it.
        const int va = lane & 3, vrow = 4 * kq + ((lane >> 2) & 3);
#pragma unroll
        for (int vb = 0; vb < VB; ++vb)
            vr_off[vb] = vrow * VROWB + (((2 * vb + (va >> 1)) ^ v_swz_dec(vrow)) * 16) + 8 * (va & 1);
    }
    char* const kst0 = kst_a[w];
    char* const kst1 = kst_b[w];
    char* const vst0 = vst_a[w];
    char* const vst1 = vst_b[w];
    auto load8 = [&](__amdgpu_buffer_rsrc_t r, uint32_t off) -> KVec {
        if constexpr (FP8) return buf_load8_nt(r, off);
        else return buf_load16_nt(r, off);
    };
    // One segment: pages [first_page, first_page + n_pg) of sequence s (L cached tokens),
    // partial result into slot `slot`.
    auto segment = [&](const int s, const int L, const int first_page, const int n_pg,
                       const int slot) __attribute__((always_inline)) {
    const int t1 = min((first_page + n_pg) * kPage, L);
    // B operand (Q^T): Q[s][h0+n][8*(4j + kq) .. +7], zero for padding columns.
    u32x4 qf[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        qf[j] = u32x4{0, 0, 0, 0};
        const int kk = (j * 4 + kq) * 8;  // element of the row read
        if (col_ok && kk / D == kn)       // a pair's column is zero in the other head's half
            qf[j] = *reinterpret_cast<const u32x4*>(q + ((size_t)s * H + head_n) * D + kk - kn * D);
    }

    float m_used = -INFINITY, l_part = 0.f;
    // P.V: this lane's chunk c of the row belongs to KV head kc of the NK; it accumulates
    // that head's G2 columns.
    const int kc = PAIR ? c / (D / 8) : 0;
    float oacc[MPV ? 1 : G2][8];
#pragma unroll
    for (int hh = 0; hh < (MPV ? 1 : G2); ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[hh][e] = 0.f;
    // MPV: O^T block vb, element i = dim 16 vb + 4 kq + i of head column n.
    f32x4 macc[MPV ? VB : 1];
#pragma unroll
    for (int vb = 0; vb < (MPV ? VB : 1); ++vb) macc[vb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // This wave's pages are first_page + w + kWaves*i, i < n_my. Lane i holds the
    // physical id of the i-th one, so no page-table load sits on the loop's critical path.
    const int n_my = w < n_pg ? (n_pg - w + kWaves - 1) / kWaves : 0;
    int pid_lane = -1;
    if (lane < n_my) pid_lane = page_table[(size_t)s * max_pages + first_page + w + kWaves * lane];
    // Let the ids arrive once, here; afterwards the register no longer counts as a pending
    // load, so reading it inside the loop does not wait for the page loads in flight.
    __asm__ volatile("" : "+v"(pid_lane));

    auto load_page = [&](int it, char* kst, KVec (&vv)[TPL], char* vst) -> bool {
        const int pid = __builtin_amdgcn_readlane(pid_lane, it);
        const bool valid = (unsigned)pid < (unsigned)num_pages;
        const size_t page_base = (size_t)(valid ? pid : 0) * kPage * tok_stride + (size_t)kvh * D;
        const auto rk = make_rsrc(static_cast<const char*>(kcache) + page_base * ES, valid ? span : 0u);
        if constexpr (MPV) {
            // The stages are rewritten only after this wave's reads of them have returned
            // (the LDS does not order a queued read before a later direct load's write).
            __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
        }
#pragma unroll
        for (int i = 0; i < KDMA; ++i) buf_load16_lds_nt(rk, kst + 1024 * i, kd_off[i], 0u);
        if constexpr (VDMA) {
            // V rows past the sequence's last token may hold anything; the descriptor ends
            // at the page's last valid row, so they arrive as zeros (0 x NaN would poison
            // the product even with a zero probability).
            const int nv = min(max(t1 - (first_page + w + kWaves * it) * kPage, 0), kPage);
            const uint32_t vspan = valid && nv > 0 ? (uint32_t)((nv - 1) * tok_stride + DR) * ES : 0u;
            const auto rv = make_rsrc(static_cast<const char*>(vcache) + page_base * ES, vspan);
#pragma unroll
            for (int i = 0; i < KDMA; ++i) buf_load16_lds_nt(rv, vst + 1024 * i, vd_off[i], 0u);
        } else {
            const auto rv = make_rsrc(static_cast<const char*>(vcache) + page_base * ES, valid ? span : 0u);
#pragma unroll
            for (int i = 0; i < TPL; ++i)
                vv[i] = load8(rv, v_off + (uint32_t)(TG * i * tok_stride) * ES);
        }
        return valid;
    };

    KVec vA[TPL], vB[TPL];
    bool okA = load_page(0, kst0, vA, vst0);   // a lane past the wave's pages holds id -1
    bool okB = false;
    // Every load of the page before this one's successor has landed: its K rows in LDS
    // (direct loads are counted by vmcnt only) and its V registers (MPV: V rows in LDS).
    auto wait_page = [&]() __attribute__((always_inline)) {
        constexpr int later = KDMA + (VDMA ? KDMA : TPL);  // loads of the page issued after it
        static_assert(later < 64, "vmcnt field");
        __builtin_amdgcn_s_waitcnt((later & 15) | ((later >> 4) << 14) | (7 << 4) | (15 << 8));
    };
    auto page_compute = [&](const char* KST, const KVec (&VV)[TPL], char* VST, const bool OK,
                            const int IT) {
        if (OK) {
            const int tok0 = (first_page + w + kWaves * IT) * kPage;
            KVec KF[KS];
#pragma unroll
            for (int j = 0; j < KS; ++j) KF[j] = *reinterpret_cast<const KVec*>(KST + kr_off[j]);

            // S^T: acc[i] = score of token 4*kq + i for head column n
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                if constexpr (FP8) {
                    const u32x2 lo = fp8x4_to_bf16x4(KF[j][0]), hi = fp8x4_to_bf16x4(KF[j][1]);
                    acc = mfma16x16x32(u32x4{lo[0], lo[1], hi[0], hi[1]}, qf[j], acc);
                } else {
                    acc = mfma16x16x32(KF[j], qf[j], acc);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tok0 + kq * 4 + i >= t1) acc[i] = -INFINITY;

            float mx = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
            mx = fmaxf(mx, shfl_xor(mx, 16));
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const float m_cand = fmaxf(m_used, mx);  // finite: a page's first token is valid
            const bool move = m_cand > m_used + tau_raw;
            const bool resc = __builtin_amdgcn_ballot_w64(move) != 0;
            float alpha = 1.f;  // alpha = 1 for unmoved heads
            if (resc) {
                const float m_new = move ? m_cand : m_used;
                alpha = move ? fast_exp2((m_used - m_new) * scale_log2) : 1.f;
                m_used = m_new;
                l_part *= alpha;
                if constexpr (!MPV)
                    if (kq == 0 && n < GH) a_lds[w][n] = alpha;
            }
            const float mb = m_used * scale_log2;
            if constexpr (MPV) {
                if constexpr (FP8) {
                    // This page's V rows into the bf16 stage (e4m3 converted exactly; zeros
                    // past the sequence): lane (tg, c) writes tokens tg + TG i, chunk c.
#pragma unroll
                    for (int i = 0; i < TPL; ++i) {
                        const int tl = tg + TG * i;
                        const bool ok = tok0 + tl < t1;
                        const u32x2 lo = fp8x4_to_bf16x4(ok ? VV[i][0] : 0u);
                        const u32x2 hi = fp8x4_to_bf16x4(ok ? VV[i][1] : 0u);
                        *reinterpret_cast<u32x4*>(VST + tl * VROWB + ((c ^ v_swz_dec(tl)) * 16)) =
                            u32x4{lo[0], lo[1], hi[0], hi[1]};
                    }
                    wave_lds_fence();  // the transposing reads take other lanes' rows
                }
                // P^T as the B operand: this lane's column n, tokens 4 kq .. 4 kq + 3 (bf16;
                // the row sum takes the unrounded values).
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = fast_exp2(fmaf(acc[i], scale_log2, -mb));
                    l_part += p[i];
                }
                const u32x2 pf = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
                if (resc) {
#pragma unroll
                    for (int vb = 0; vb < VB; ++vb) macc[vb] *= alpha;  // column n is this lane's
                }
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    const u32x2 a = prefill::lds_read_tr(VST + vr_off[vb]);
                    macc[vb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        __builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, pf), macc[vb],
                        0, 0, 0);
                }
                return;
            }
            float pq[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(fmaf(acc[i], scale_log2, -mb));
                l_part += p;  // the row sum takes the unrounded values
                pq[i] = p;
                if constexpr (!DOT)
                    if (n < GH) p_lds[w][kq * 4 + i][n] = p;
            }
            if constexpr (DOT) {
                if (n < GH) {
                    p2_lds[w][2 * kq][n] = pack_bf16x2(pq[0], pq[2]);
                    p2_lds[w][2 * kq + 1][n] = pack_bf16x2(pq[1], pq[3]);
                }
            }
            wave_lds_fence();

            if (resc) {
#pragma unroll
                for (int hh = 0; hh < G2; ++hh) {
                    const float a = a_lds[w][kc * G2 + hh];
#pragma unroll
                    for (int e = 0; e < 8; ++e) oacc[hh][e] *= a;
                }
            }
            {
                // Tokens a = tg + TG (2 ip) and b = a + TG (the lane's VV[2 ip], VV[2 ip + 1];
                // with pairs 4 ip + tg and 4 ip + tg + 2): each dim's two values become one
                // bf16 pair, and one v_dot2c per (dim, head) adds p_a v_a + p_b v_b to the
                // fp32 accumulator.
#pragma unroll
                for (int ip = 0; ip < TPL / 2; ++ip) {
                    const int ta = tg + TG * (2 * ip);
                    const bool oka = tok0 + ta < t1, okb = tok0 + ta + TG < t1;  // past the
                    uint32_t wa[4], wb[4];  // sequence: zeros (slots may hold anything)
                    if constexpr (FP8) {
                        const u32x2 a0 = fp8x4_to_bf16x4(oka ? VV[2 * ip][0] : 0u);
                        const u32x2 a1 = fp8x4_to_bf16x4(oka ? VV[2 * ip][1] : 0u);
                        const u32x2 b0 = fp8x4_to_bf16x4(okb ? VV[2 * ip + 1][0] : 0u);
                        const u32x2 b1 = fp8x4_to_bf16x4(okb ? VV[2 * ip + 1][1] : 0u);
                        wa[0] = a0[0]; wa[1] = a0[1]; wa[2] = a1[0]; wa[3] = a1[1];
                        wb[0] = b0[0]; wb[1] = b0[1]; wb[2] = b1[0]; wb[3] = b1[1];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            wa[e] = oka ? VV[2 * ip][e] : 0u;
                            wb[e] = okb ? VV[2 * ip + 1][e] : 0u;
                        }
                    }
                    uint32_t pp[G2];  // bf16 pairs (p_a, p_b) of the lane's heads
                    if constexpr (DOT) {
                        // (element by element into the array: this compiler bit-casts a vector
                        // element taken in place as element 0)
                        const u32x4 p4 = *reinterpret_cast<const u32x4*>(&p2_lds[w][2 * ip + tg][kc * G2]);
#pragma unroll
                        for (int hh = 0; hh < G2; ++hh) pp[hh] = p4[hh];
                    } else {
#pragma unroll
                        for (int hh = 0; hh < G2; ++hh)
                            pp[hh] = pack_bf16x2(p_lds[w][ta][kc * G2 + hh],
                                                 p_lds[w][ta + TG][kc * G2 + hh]);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // (a, b) of dims 2e and 2e + 1: low halves, high halves
                        const uint32_t lo = __builtin_amdgcn_perm(wb[e], wa[e], 0x05040100u);
                        const uint32_t hi = __builtin_amdgcn_perm(wb[e], wa[e], 0x07060302u);
#pragma unroll
                        for (int hh = 0; hh < G2; ++hh) {
                            const bf16x2 ph = __builtin_bit_cast(bf16x2, pp[hh]);
                            oacc[hh][2 * e] = __builtin_amdgcn_fdot2_f32_bf16(
                                __builtin_bit_cast(bf16x2, lo), ph, oacc[hh][2 * e], false);
                            oacc[hh][2 * e + 1] = __builtin_amdgcn_fdot2_f32_bf16(
                                __builtin_bit_cast(bf16x2, hi), ph, oacc[hh][2 * e + 1], false);
                        }
                    }
                }
                wave_lds_fence();
            }
        }
    };
    for (int it = 0; it < n_my; it += 2) {
        okB = load_page(it + 1, kst1, vB, vst1);
        wait_page();
        page_compute(kst0, vA, vst0, okA, it);
        okA = load_page(it + 2, kst0, vA, vst0);
        wait_page();
        page_compute(kst1, vB, vst1, okB, it + 1);
    }
    // The loop ends with two pages' loads still in flight (past the wave's last page: zero
    // descriptors, but their LDS writes land in the stages reused below).
    __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));

    // ---- reduce within the wave, then across the 4 waves ----
    float l = l_part;
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (kq == 0 && n < GH) {
        red_m[w][n] = m_used;
        red_l[w][n] = l;
    }
    if constexpr (MPV) {
        // The matrix unit summed over the tokens already: lane (n, kq) holds dims
        // 16 vb + 4 kq + i of head column n.
        if (n < nheads) {
            float* ro = red_o_row(w, n);
#pragma unroll
            for (int vb = 0; vb < VB; ++vb)
                *reinterpret_cast<f32x4*>(ro + 16 * vb + 4 * kq) = macc[vb];
        }
    } else {
#pragma unroll
        for (int hh = 0; hh < G2; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = oacc[hh][e];
#pragma unroll
                for (int msk = CH; msk < 64; msk <<= 1) x += shfl_xor(x, msk);
                oacc[hh][e] = x;
            }
        if (tg == 0) {
#pragma unroll
            for (int hh = 0; hh < G2; ++hh) {
                float* ro = red_o_row(w, kc * G2 + hh) + (c % (D / 8)) * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) ro[e] = oacc[hh][e];
            }
        }
    }
    __syncthreads();

    for (int idx = tid; idx < (PAIR ? GH : nheads) * D; idx += 256) {
        const int hh = idx / D, dd = idx % D;  // column, dim
        if (PAIR && hh % G2 >= g) continue;    // a pair's padding column
        // The column's scales (a pair's columns come from two KV heads).
        // (bf16 caches have no scale arrays: their columns share scale_log2 and v_sc = 1.)
        float sc = scale_log2, vs = v_sc;
        if constexpr (PAIR && FP8) {
            sc = scale_log2_in * k_scale[kvh + hh / G2];
            vs = v_scale[kvh + hh / G2];
        }
        const int head = PAIR ? (kvh + hh / G2) * g + hh % G2 : h0 + hh;
        float M = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, red_m[ww][hh]);
        float lsum = 0.f, acc = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) {
                const float mw = red_m[ww][hh];  // -inf for a wave that saw no token
                const float f = mw == -INFINITY ? 0.f : fast_exp2((mw - M) * sc);
                lsum = fmaf(f, red_l[ww][hh], lsum);
                acc = fmaf(f, red_o_row(ww, hh)[dd], acc);
            }
        }
        const size_t row = ((size_t)s * H + head) * max_slots + slot;
        o_part[row * D + dd] = M != -INFINITY ? acc / lsum * vs : 0.f;
        if (dd == 0)
            lse_part[row] = M != -INFINITY ? M * sc + fast_log2(lsum) : -INFINITY;
    }
    __syncthreads();  // the next segment's loads overwrite the merge buffers
    };

    // ---- the work-group's range of pages, and the segments in it ----
    // Pages of all sequences end to end (per KV head): sequence s holds [S_s, S_s + P_s).
    // Every wave computes the same plan from the lengths.
    // Work-groups in use: the target, at least one per non-empty sequence (many short
    // sequences then get a range each instead of ranges cut into several short pieces,
    // each restarting the page pipeline), and as many as keep R <= kMaxRangePages (at most
    // the launched ones, which suffice for the longest possible cache); the rest return.
    // Up to 64 sequences every work-group works this out from the lengths (one load per
    // lane); beyond, decode_plan_kernel has done it once and also recorded where each
    // work-group's range starts, so no work-group reads every length.
    int P_tot, n_wg, R, c_first = 0, base = 0;  // base: pages of the sequences before c_first
    if (plan != nullptr) {
        P_tot = plan[0];
        n_wg = plan[1];
        R = plan[2];
        if ((int)blockIdx.y >= n_wg || (int)blockIdx.y * R >= P_tot) return;  // uniform
        c_first = plan[4 + 2 * blockIdx.y];
        base = plan[5 + 2 * blockIdx.y];
    } else {
        const int Ls = lane < num_seqs ? min(max(seq_lens[lane], 0), max_seq_len) : 0;
        int p = (Ls + kPage - 1) / kPage;
#pragma unroll
        for (int msk = 1; msk < 64; msk <<= 1) p += __shfl_xor(p, msk, 64);
        P_tot = __builtin_amdgcn_readfirstlane(p);
        const int n_live = __builtin_popcountll(__builtin_amdgcn_ballot_w64(Ls > 0));
        n_wg = min((int)gridDim.y,
                   max(max(wg_target, n_live), (P_tot + kMaxRangePages - 1) / kMaxRangePages));
        R = max(rmin, (P_tot + n_wg - 1) / n_wg);
        if ((int)blockIdx.y * R >= P_tot) return;  // uniform: nothing left for this one
    }
    const int g0 = (int)blockIdx.y * R;
    const int g1 = min(g0 + R, P_tot);
    for (int c0 = c_first; c0 < num_seqs && base < g1; c0 += 64) {
        const int Ls = c0 + lane < num_seqs ? min(max(seq_lens[c0 + lane], 0), max_seq_len) : 0;
        const int Ps = (Ls + kPage - 1) / kPage;
        int x = Ps;  // inclusive prefix sum over the lanes
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        const int S = base + x - Ps;
        unsigned long long segs = __builtin_amdgcn_ballot_w64(Ps > 0 && S < g1 && S + Ps > g0);
        while (segs) {
            const int ln = __builtin_ctzll(segs);
            segs &= segs - 1;
            const int Ss = __builtin_amdgcn_readlane(S, ln);
            const int Pq = __builtin_amdgcn_readlane(Ps, ln);
            const int a = max(g0, Ss) - Ss, b = min(g1, Ss + Pq) - Ss;
            const int slot = (int)blockIdx.y - Ss / R;
            // The first work-group of a sequence records how many slots it has.
            if (slot == 0 && tid == 0) n_slots[c0 + ln] = (Ss + Pq - 1) / R - Ss / R + 1;
            segment(c0 + ln, __builtin_amdgcn_readlane(Ls, ln), a, b - a, slot);
        }
        base += __builtin_amdgcn_readlane(x, 63);
    }
}

// Plan for more than 64 sequences (the split kernel's work-group rule, worked out once):
// plan[0] = all pages (per KV head), plan[1] = work-groups in use, plan[2] = R (pages per
// range); for work-group j < plan[1] whose range starts before the end, plan[4 + 2j] = the
// sequence holding its first page j R and plan[5 + 2j] = that sequence's first page.
// Sequence s, holding pages [S_s, S_s + P_s), is that sequence for every j with
// S_s <= j R < S_s + P_s, so a second pass over the lengths fills the table with no search.
// One work-group of 1024 threads walks the lengths 1024 at a time.
__device__ __forceinline__ void plan_prefix(const int32_t* __restrict__ seq_lens, int num_seqs,
                                            int max_seq_len, int c0, int carry, int* wave_sums,
                                            int& L, int& P, int& S, int& chunk_total,
                                            int& chunk_live) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int s = c0 + tid;
    L = s < num_seqs ? min(max(seq_lens[s], 0), max_seq_len) : 0;
    P = (L + kPage - 1) / kPage;
    int x = P;  // inclusive prefix sum over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    const unsigned long long live_mask = __builtin_amdgcn_ballot_w64(L > 0);  // all lanes vote
    if (lane == 63) wave_sums[w] = x;
    if (lane == 0) wave_sums[16 + w] = __builtin_popcountll(live_mask);
    __syncthreads();
    int before = 0;
    chunk_total = 0;
    chunk_live = 0;
    for (int i = 0; i < 16; ++i) {
        before += i < w ? wave_sums[i] : 0;
        chunk_total += wave_sums[i];
        chunk_live += wave_sums[16 + i];
    }
    S = carry + before + x - P;
    __syncthreads();  // the sums are rewritten by the next 1024
}

__global__ __launch_bounds__(1024) void decode_plan_kernel(const int32_t* __restrict__ seq_lens,
                                                           int num_seqs, int max_seq_len,
                                                           int wg_target, int wg_launched,
                                                           int rmin, int* __restrict__ plan) {
    __shared__ int wave_sums[32];
    int L, P, S, total, live_c;
    int P_tot = 0, live = 0;
    for (int c0 = 0; c0 < num_seqs; c0 += 1024) {
        plan_prefix(seq_lens, num_seqs, max_seq_len, c0, P_tot, wave_sums, L, P, S, total, live_c);
        P_tot += total;
        live += live_c;
    }
    const int n_wg = min(wg_launched,
                         max(max(wg_target, live), (P_tot + kMaxRangePages - 1) / kMaxRangePages));
    const int R = max(rmin, (P_tot + n_wg - 1) / n_wg);
    if (threadIdx.x == 0) {
        plan[0] = P_tot;
        plan[1] = n_wg;
        plan[2] = R;
        plan[3] = live;
    }
    int carry = 0;
    for (int c0 = 0; c0 < num_seqs; c0 += 1024) {
        plan_prefix(seq_lens, num_seqs, max_seq_len, c0, carry, wave_sums, L, P, S, total, live_c);
        carry += total;
        if (P > 0)
            for (int j = (S + R - 1) / R; j * R < S + P && j < n_wg; ++j) {
                plan[4 + 2 * j] = c0 + (int)threadIdx.x;
                plan[5 + 2 * j] = S;
            }
    }
}

// Merge the slots of each (sequence, head): LSE = log2 sum_k 2^lse_k (relative to the
// largest), O = sum_k 2^(lse_k - LSE) O_k. One wave per (sequence, head), kCombineHeads
// heads per work-group. The slot statistics are spread over the lanes (one slot per
// lane, wave reductions for the max and the sum); each lane then owns D/64 output dims and
// walks the slots with eight partial rows in flight, the weights broadcast from the lane
// that holds them. The wave issues its first loads before it knows the slot count: the
// length, the count, one slot statistic per lane and the first kCombinePre partial rows,
// all inside the workspace whatever the count (a head's max_slots >= 2 rows). What lies
// past the sequence's own slots (stale or never written) is only ever dropped by a select,
// never multiplied, so the launch waits for one round trip to memory before its arithmetic
// instead of three.
constexpr int kCombineHeads = 4;
constexpr int kCombinePre = 8;
template <int D>
__global__ __launch_bounds__(64 * kCombineHeads) void decode_combine_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    const int* __restrict__ n_slots, const int32_t* __restrict__ seq_lens,
    uint16_t* __restrict__ o, float* __restrict__ lse, int H, int max_seq_len, int max_slots) {
    constexpr int PER = D / 64;  // output dims per lane (2 or 1)
    const int s = blockIdx.y, lane = threadIdx.x & 63;
    const int h = blockIdx.x * kCombineHeads + (threadIdx.x >> 6);
    if (h >= H) return;  // uniform per wave
    const size_t row = (size_t)s * H + h;
    const float* lp = lse_part + row * max_slots;
    const float* op = o_part + row * max_slots * D + lane * PER;

    const int len = seq_lens[s];
    const int ns_stored = n_slots[s];  // in range for every s; not written for an empty sequence
    const float lp0 = lane < max_slots ? lp[lane] : -INFINITY;
    float x0[kCombinePre][PER];
#pragma unroll
    for (int u = 0; u < kCombinePre; ++u) {
#pragma unroll
        for (int e = 0; e < PER; ++e) x0[u][e] = 0.f;
        if (u < max_slots) {  // uniform
            const float* src = op + (size_t)u * D;
            if constexpr (PER == 2) {
                const f32x2 v2 = *reinterpret_cast<const f32x2*>(src);
                x0[u][0] = v2[0];
                x0[u][1] = v2[1];
            } else {
                x0[u][0] = src[0];
            }
        }
    }
    const int L = min(max(len, 0), max_seq_len);
    const int ns = L > 0 ? ns_stored : 0;  // no slot was written for an empty sequence

    float m = lane < ns ? lp0 : -INFINITY;
    for (int k = lane + 64; k < ns; k += 64) m = fmaxf(m, lp[k]);
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) m = fmaxf(m, shfl_xor(m, msk));
    const float M = m;  // -inf: no slot holds a token (L = 0)

    float out[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = 0.f;
    float wsum = 0.f;
    if (M != -INFINITY) {
        for (int kb = 0; kb < ns; kb += 64) {
            // weight of slot kb + lane (0 past the last slot)
            const float fl = kb + lane < ns ? fast_exp2((kb == 0 ? lp0 : lp[kb + lane]) - M) : 0.f;
            wsum += fl;
            const int cnt = min(64, ns - kb);
            auto fw = [&](int kk) {
                return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), kk));
            };
            int kk = 0;
            if (kb == 0) {
                // the rows loaded up front: slots 0 .. min(cnt, kCombinePre) - 1
#pragma unroll
                for (int u = 0; u < kCombinePre; ++u) {
                    if (u < cnt) {  // uniform
                        const float f = fw(u);
#pragma unroll
                        for (int e = 0; e < PER; ++e) out[e] = fmaf(f, x0[u][e], out[e]);
                    }
                }
                kk = min(cnt, kCombinePre);
            }
            for (; kk + 8 <= cnt; kk += 8) {
                float x[8][PER];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float* src = op + (size_t)(kb + kk + u) * D;
                    if constexpr (PER == 2) {
                        const f32x2 v2 = *reinterpret_cast<const f32x2*>(src);
                        x[u][0] = v2[0];
                        x[u][1] = v2[1];
                    } else {
                        x[u][0] = src[0];
                    }
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float f = fw(kk + u);
#pragma unroll
                    for (int e = 0; e < PER; ++e) out[e] = fmaf(f, x[u][e], out[e]);
                }
            }
            for (; kk < cnt; ++kk) {
                const float f = fw(kk);
                const float* src = op + (size_t)(kb + kk) * D;
#pragma unroll
                for (int e = 0; e < PER; ++e) out[e] = fmaf(f, src[e], out[e]);
            }
        }
#pragma unroll
        for (int msk = 1; msk < 64; msk <<= 1) wsum += shfl_xor(wsum, msk);
        const float inv = 1.f / wsum;
#pragma unroll
        for (int e = 0; e < PER; ++e) out[e] *= inv;
    }
    uint16_t* orow = o + row * D + lane * PER;
    if constexpr (PER == 2) {
        *reinterpret_cast<uint32_t*>(orow) = pack_bf16x2(out[0], out[1]);
    } else {
        orow[0] = (uint16_t)(pack_bf16x2(out[0], 0.f) & 0xffffu);
    }
    if (lse != nullptr && lane == 0)
        lse[row] = M != -INFINITY ? (M + fast_log2(wsum)) * kLn2 : -INFINITY;
}

// Workspace: o_part [num_seqs, H, max_slots, D] fp32, lse_part [num_seqs, H, max_slots]
// fp32, n_slots [num_seqs] int32, plan [4 + 2 x the launched work-groups] int32.
struct DecodeWorkspace {
    float* o_part;
    float* lse_part;
    int* n_slots;
    int* plan;
};
DecodeWorkspace decode_workspace(void* ws, int num_seqs, int H, int d, int max_slots) {
    const size_t rows = (size_t)num_seqs * H * max_slots;
    float* o_part = static_cast<float*>(ws);
    float* lse_part = o_part + rows * d;
    int* n_slots = reinterpret_cast<int*>(lse_part + rows);
    return {o_part, lse_part, n_slots, n_slots + num_seqs};
}

// Work-groups aimed at: one round of resident ones (two for an fp8 cache on the VALU
// kernel, whose ranges take half the time; one on the matrix-unit kernel: 64 x
// U{512..8192}, H32 Hkv2, 59.9 -> 52.2 us) shared by the (KV head, head group) pairs: 256
// CUs (MI355X) times the
// work-groups a CU holds. VALU P.V: by register use, 3 for 4 heads per group, 2 for 8, 1
// for 16. Matrix-unit P.V: by LDS (four K/V page stages per wave), 2 for d = 128 (66 KiB
// each), 4 for d = 64, 3 for an e4m3 cache (its K stages are half the size: 49 KiB).
// (Fixed numbers: no runtime query precedes the launch.)
constexpr int kCUs = 256;
int decode_target(int GH, bool mma, int groups, int d, bool fp8) {
    const int per_cu = mma ? (fp8 ? 3 : d == 128 ? 2 : 4) : GH == 4 ? 3 : GH == 8 ? 2 : 1;
    return std::max(1, per_cu * kCUs * (fp8 && !mma ? 2 : 1) / groups);
}
// Pairs: one round of the pair kernel's work-groups per CU (3 for bf16 with d = 64, else 2,
// by their register use) over the KV head pairs; two or four rounds were slower.
int decode_target_pair(int pairs, bool fp8, int d) {
    const int per_cu = !fp8 && d == 64 ? 3 : 2;
    return std::max(1, per_cu * kCUs / pairs);
}
// The most work-groups per (KV head, head group) a launch can have, for any head count or
// cache type: sizes the plan in the workspace.
int decode_max_rows(const DecodePlan& plan, int num_seqs) {
    return std::max(std::max(3 * kCUs * 2, plan.min_wgs), num_seqs);
}

template <int D, int GH, bool FP8, bool PAIR = false, bool MMA = false>
hipError_t launch_split(const void* q, const void* kc, const void* vc, const int32_t* pt,
                        const int32_t* sl, const DecodeWorkspace& ws, const DecodePlan& plan,
                        int target, int rows, int num_seqs, int H, int Hkv, int g, int n_hg,
                        int num_pages, int max_pages, int max_seq_len, float scale,
                        ScalePtr<FP8> k_scale, ScalePtr<FP8> v_scale, hipStream_t stream) {
    const float scale_log2 = scale * kLog2e;
    // KV heads vary fastest: the work-groups covering one page range are dispatched
    // together, so each physical page (all KV heads of 16 slots, contiguous) is read by
    // concurrently running work-groups.
    dim3 grid(Hkv * n_hg / (PAIR ? 2 : 1), rows);
    hipLaunchKernelGGL((decode_split_kernel<D, GH, FP8, PAIR, MMA>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), kc, vc, pt, sl, ws.o_part, ws.lse_part,
                       ws.n_slots, num_seqs > 64 ? ws.plan : nullptr, num_seqs, H, Hkv, g, n_hg,
                       num_pages, max_pages, max_seq_len,
                       plan.rmin, plan.max_slots, target, scale_log2, k_scale, v_scale);
    return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_split_d(int GH, bool pair, bool mma, const void* q, const void* kc, const void* vc,
                          const int32_t* pt, const int32_t* sl, const DecodeWorkspace& ws,
                          const DecodePlan& plan, int target, int rows, int num_seqs, int H,
                          int Hkv, int g, int n_hg, int num_pages, int max_pages,
                          int max_seq_len, float scale, ScalePtr<FP8> ks, ScalePtr<FP8> vs,
                          hipStream_t stream) {
    if constexpr (D * (FP8 ? 1 : 2) == 128 || (!FP8 && D == 128))
        if (pair)
            return launch_split<D, 8, FP8, true>(q, kc, vc, pt, sl, ws, plan, target, rows,
                                                  num_seqs, H, Hkv, g, n_hg, num_pages,
                                                  max_pages, max_seq_len, scale, ks, vs, stream);
    if constexpr (!FP8 || D == 128)
        if (mma) {
            if (GH == 4)
                return launch_split<D, 4, FP8, false, true>(
                    q, kc, vc, pt, sl, ws, plan, target, rows, num_seqs, H, Hkv, g, n_hg,
                    num_pages, max_pages, max_seq_len, scale, ks, vs, stream);
            if (GH == 8)
                return launch_split<D, 8, FP8, false, true>(
                    q, kc, vc, pt, sl, ws, plan, target, rows, num_seqs, H, Hkv, g, n_hg,
                    num_pages, max_pages, max_seq_len, scale, ks, vs, stream);
            return launch_split<D, 16, FP8, false, true>(
                q, kc, vc, pt, sl, ws, plan, target, rows, num_seqs, H, Hkv, g, n_hg, num_pages,
                max_pages, max_seq_len, scale, ks, vs, stream);
        }
    if (GH == 4)
        return launch_split<D, 4, FP8>(q, kc, vc, pt, sl, ws, plan, target, rows, num_seqs, H, Hkv, g, n_hg,
                                       num_pages, max_pages, max_seq_len, scale, ks, vs, stream);
    if (GH == 8)
        return launch_split<D, 8, FP8>(q, kc, vc, pt, sl, ws, plan, target, rows, num_seqs, H, Hkv, g, n_hg,
                                       num_pages, max_pages, max_seq_len, scale, ks, vs, stream);
    return launch_split<D, 16, FP8>(q, kc, vc, pt, sl, ws, plan, target, rows, num_seqs, H, Hkv, g, n_hg,
                                    num_pages, max_pages, max_seq_len, scale, ks, vs, stream);
}

}  // namespace

int decode_split_tokens(int num_seqs, int max_seq_len) {
    return decode_plan(num_seqs, max_seq_len).rmin * kPage;
}

int decode_min_work_groups(int num_seqs, int max_seq_len) {
    return decode_plan(num_seqs, max_seq_len).min_wgs;
}

size_t decode_workspace_bytes(int num_seqs, int H, int d, int max_seq_len) {
    const DecodePlan plan = decode_plan(num_seqs, max_seq_len);
    const size_t rows = (size_t)num_seqs * H * plan.max_slots;
    return rows * (size_t)d * sizeof(float) + rows * sizeof(float) +
           (size_t)num_seqs * sizeof(int) +
           (4 + 2 * (size_t)decode_max_rows(plan, num_seqs)) * sizeof(int);
}

hipError_t launch_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* page_table, const int32_t* seq_lens, void* o,
                               float* lse, int num_seqs, int H, int Hkv, int d, int num_pages,
                               int max_pages_per_seq, int max_seq_len, float scale,
                               void* workspace, hipStream_t stream, DecodeCache cache,
                               const float* k_scale, const float* v_scale) {
    const bool fp8 = cache == DecodeCache::kFp8;
    if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return hipErrorInvalidValue;
    const int g = H / Hkv;
    const int GH = g <= 4 ? 4 : g <= 8 ? 8 : 16;
    const int n_hg = g <= 16 ? 1 : g / 16;
    const DecodePlan plan = decode_plan(num_seqs, max_seq_len);
    const DecodeWorkspace ws = decode_workspace(workspace, num_seqs, H, d, plan.max_slots);

    // An even KV head count and at most 4 query heads per KV head: KV heads are read in
    // pairs (128-byte rows of an e4m3 cache with d = 128 or a bf16 one with d = 64 become
    // 256-byte rows; bf16 rows with d = 128 become 512-byte rows).
    // Small batches (under 32 sequences) keep single heads: their work-groups are few, and
    // pairs would halve them (1 x 8192 tokens, H32 Hkv8 d128: 15.3 us single, 16.6 paired).
    const bool pair = (d * (fp8 ? 1 : 2) == 128 || (!fp8 && d == 128)) && Hkv % 2 == 0 &&
                      g <= 4 && num_seqs >= 32;
    // Single KV heads of a bf16 cache: P.V on the matrix unit, except for groups of up to 4
    // heads over 32 or more sequences, where the VALU kernel's third resident work-group per
    // CU (the matrix-unit kernel's V stages leave room for two) reads faster (measured when
    // the VALU P.V still ran on fp32 FMAs: 64 x U{512..8192}, H28 Hkv7: 177.6 us on the VALU,
    // 200.4 us on the matrix unit; 16 x 1024, H32 Hkv8: 22.7 vs 16.9 us; 64 x U{512..8192},
    // H32 Hkv2: 93.2 vs 65.2 us). An e4m3 cache with d = 128
    // follows the same rule (64 x U{512..8192}: H32 Hkv4 84.7 -> 74.4 us, H32 Hkv2 89.7 ->
    // 59.6 us against the VALU kernel, which holds every head's accumulators; 1 x 8192, H32
    // Hkv8: 11.8 -> 10.9 us).
    const bool mma = !pair && (!fp8 || d == 128) && (GH >= 8 || num_seqs < 32);
    const int target = pair ? decode_target_pair(Hkv / 2, fp8, d)
                            : decode_target(GH, mma, Hkv * n_hg, d, fp8);
    const int rows = std::max(std::max(target, plan.min_wgs), num_seqs);  // <= decode_max_rows

    hipError_t e;
    if (num_seqs > 64) {
        hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, seq_lens,
                           num_seqs, max_seq_len, target, rows, plan.rmin, ws.plan);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (d == 128)
        e = fp8 ? launch_split_d<128, true>(GH, pair, mma, q, k_cache, v_cache, page_table, seq_lens, ws,
                                            plan, target, rows, num_seqs, H, Hkv, g, n_hg, num_pages,
                                            max_pages_per_seq, max_seq_len, scale, k_scale,
                                            v_scale, stream)
                : launch_split_d<128, false>(GH, pair, mma, q, k_cache, v_cache, page_table, seq_lens, ws,
                                             plan, target, rows, num_seqs, H, Hkv, g, n_hg, num_pages,
                                             max_pages_per_seq, max_seq_len, scale, nullptr,
                                             nullptr, stream);
    else
        e = fp8 ? launch_split_d<64, true>(GH, pair, mma, q, k_cache, v_cache, page_table, seq_lens, ws,
                                           plan, target, rows, num_seqs, H, Hkv, g, n_hg, num_pages,
                                           max_pages_per_seq, max_seq_len, scale, k_scale,
                                           v_scale, stream)
                : launch_split_d<64, false>(GH, pair, mma, q, k_cache, v_cache, page_table, seq_lens, ws,
                                            plan, target, rows, num_seqs, H, Hkv, g, n_hg, num_pages,
                                            max_pages_per_seq, max_seq_len, scale, nullptr,
                                            nullptr, stream);
    if (e != hipSuccess) return e;
    dim3 grid((H + kCombineHeads - 1) / kCombineHeads, num_seqs);
    if (d == 128)
        hipLaunchKernelGGL(decode_combine_kernel<128>, grid, dim3(64 * kCombineHeads), 0, stream,
                           ws.o_part, ws.lse_part, ws.n_slots, seq_lens,
                           static_cast<uint16_t*>(o), lse, H, max_seq_len, plan.max_slots);
    else
        hipLaunchKernelGGL(decode_combine_kernel<64>, grid, dim3(64 * kCombineHeads), 0, stream,
                           ws.o_part, ws.lse_part, ws.n_slots, seq_lens,
                           static_cast<uint16_t*>(o), lse, H, max_seq_len, plan.max_slots);
    return hipGetLastError();
}

}  // namespace kvfa
