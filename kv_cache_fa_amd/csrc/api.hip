// C ABI of libkvfa.so (declared in include/kvfa.h): argument validation and dispatch.
// Validation runs entirely on the host and returns before any HIP call, so a rejected
// call enqueues nothing and touches no output.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "kvfa.h"
#include "launch.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Status of a launch. With KVFA_DEBUG set in the environment, a HIP failure is also
// described on stderr (the C status only says that HIP failed).
int hip_status(hipError_t e, const char* fn) {
    if (e == hipSuccess) return FA_OK;
    if (getenv("KVFA_DEBUG") != nullptr)
        fprintf(stderr, "kvfa: %s: HIP error %d (%s): %s\n", fn, (int)e, hipGetErrorName(e),
                hipGetErrorString(e));
    return FA_ERR_HIP;
}

// Shared checks of the two prefill entry points.
int check_prefill(const void* q, const void* k, const void* v, const void* o, const void* lse,
                  int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                  size_t elem) {
    if (!q || !k || !v || !o) return FA_ERR_INVALID;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return FA_ERR_INVALID;
    if (lse && !aligned(lse, 4)) return FA_ERR_INVALID;
    if (B < 1 || H < 1 || Hkv < 1 || Nq < 1 || Nk < 1) return FA_ERR_INVALID;
    if (H % Hkv != 0) return FA_ERR_INVALID;
    if (causal && Nq > Nk) return FA_ERR_INVALID;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    // One head's slice is addressed with 32-bit byte offsets.
    const unsigned long long lim = 1ull << 31;
    if ((unsigned long long)Nk * d * elem >= lim || (unsigned long long)Nq * d * elem >= lim)
        return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

int decode_checked(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* page_table, const int32_t* seq_lens, int page_size, void* o,
                   float* lse, int num_seqs, int H, int Hkv, int d, int num_pages,
                   int max_pages_per_seq, int max_seq_len, float scale, void* workspace,
                   size_t workspace_bytes, hipStream_t stream, const float* k_scale,
                   const float* v_scale);

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int Hkv, int Nq, int Nk, int d, int causal, float scale, hipStream_t stream) {
    int st = check_prefill(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal, scale, 2);
    if (st != FA_OK) return st;
    const unsigned long long n_wg = (unsigned long long)((Nq + 127) / 128) * B * H;
    if (n_wg >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
    hipError_t e = kvfa::launch_fwd_bf16(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal != 0, scale,
                                         stream);
    return hip_status(e, "fa_fwd");
}

int fa_fwd_two_pass(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                    hipStream_t stream) {
    if (!lse) return FA_ERR_INVALID;  // carries the row statistics between the passes
    int st = check_prefill(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal, scale, 2);
    if (st != FA_OK) return st;
    const unsigned long long n_wg = (unsigned long long)((Nq + 127) / 128) * B * H;
    if (n_wg >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
    hipError_t e = kvfa::launch_fwd_bf16_two_pass(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d,
                                                  causal != 0, scale,
                                                  stream);
    return hip_status(e, "fa_fwd_two_pass");
}

int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int Hkv, int Nq, int Nk, int d, int window_left, int window_right,
                  float scale, hipStream_t stream) {
    // The window is placed at each query's position Nk - Nq + i, so Nq <= Nk as for causal.
    int st = check_prefill(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, 1, scale, 2);
    if (st != FA_OK) return st;
    if (window_left < -1 || window_right < -1) return FA_ERR_INVALID;
    const unsigned long long n_wg = (unsigned long long)((Nq + 127) / 128) * B * H;
    if (n_wg >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
    hipError_t e = kvfa::launch_fwd_bf16_window(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d,
                                                window_left, window_right, scale,
                                                stream);
    return hip_status(e, "fa_fwd_window");
}

int fa_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                int H, int Hkv, int Nq, int Nk, int d, int causal, float scale, hipStream_t stream) {
    int st = check_prefill(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal, scale, 4);
    if (st != FA_OK) return st;
    if (H > 65535 || B > 65535) return FA_ERR_UNSUPPORTED;
    hipError_t e = kvfa::launch_fwd_fp32(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal != 0, scale,
                                         stream);
    return hip_status(e, "fa_fwd_fp32");
}

int fa_decode_paged_split_tokens(int num_seqs, int max_seq_len, int page_size) {
    if (num_seqs < 1 || max_seq_len < 1 || page_size != 16) return 0;
    return kvfa::decode_split_tokens(num_seqs, max_seq_len);
}

size_t fa_decode_paged_workspace_size(int num_seqs, int H, int d, int max_seq_len,
                                      int page_size) {
    if (num_seqs < 1 || H < 1 || max_seq_len < 1 || page_size != 16) return 0;
    if (d != 64 && d != 128) return 0;
    return kvfa::decode_workspace_bytes(num_seqs, H, d, max_seq_len);
}

int fa_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* page_table, const int32_t* seq_lens, int page_size, void* o,
                    float* lse, int num_seqs, int H, int Hkv, int d, int num_pages,
                    int max_pages_per_seq, int max_seq_len, float scale, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
    return decode_checked(q, k_cache, v_cache, page_table, seq_lens, page_size, o, lse, num_seqs,
                          H, Hkv, d, num_pages, max_pages_per_seq, max_seq_len, scale, workspace,
                          workspace_bytes, stream, nullptr, nullptr);
}

}  // extern "C"

namespace {
// Checks of the decode arguments other than the workspace (host only, no HIP call).
int decode_args_status(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* page_table, const int32_t* seq_lens, int page_size,
                       void* o, float* lse, int num_seqs, int H, int Hkv, int d,
                       int num_pages, int max_pages_per_seq, int max_seq_len, float scale) {
    if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !o) return FA_ERR_INVALID;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
        !aligned(page_table, 4) || !aligned(seq_lens, 4))
        return FA_ERR_INVALID;
    if (lse && !aligned(lse, 4)) return FA_ERR_INVALID;
    if (num_seqs < 1 || H < 1 || Hkv < 1 || num_pages < 1 || max_pages_per_seq < 1 ||
        max_seq_len < 1)
        return FA_ERR_INVALID;
    if (H % Hkv != 0) return FA_ERR_INVALID;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID;
    if (page_size != 16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
    if ((long long)max_pages_per_seq * page_size < max_seq_len) return FA_ERR_INVALID;
    const int g = H / Hkv;
    if (g > 16 && g % 16 != 0) return FA_ERR_UNSUPPORTED;
    if (num_seqs > 65535 || (long long)Hkv * (g > 16 ? g / 16 : 1) > 65535)
        return FA_ERR_UNSUPPORTED;
    // Pages over all sequences are counted in 32 bits; one grid row per work-group range.
    if ((long long)num_seqs * ((max_seq_len + page_size - 1) / page_size) >= (1LL << 30) ||
        kvfa::decode_min_work_groups(num_seqs, max_seq_len) > 65535)
        return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

int decode_checked(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* page_table, const int32_t* seq_lens, int page_size, void* o,
                   float* lse, int num_seqs, int H, int Hkv, int d, int num_pages,
                   int max_pages_per_seq, int max_seq_len, float scale, void* workspace,
                   size_t workspace_bytes, hipStream_t stream, const float* k_scale,
                   const float* v_scale) {
    const int st = decode_args_status(q, k_cache, v_cache, page_table, seq_lens, page_size, o,
                                      lse, num_seqs, H, Hkv, d, num_pages, max_pages_per_seq,
                                      max_seq_len, scale);
    if (st != FA_OK) return st;
    if (!workspace || !aligned(workspace, 16)) return FA_ERR_INVALID;
    if (workspace_bytes < kvfa::decode_workspace_bytes(num_seqs, H, d, max_seq_len))
        return FA_ERR_INVALID;
    // The cache type travels with the scales: an e4m3 cache has both, a bf16 one neither.
    if ((k_scale == nullptr) != (v_scale == nullptr)) return FA_ERR_INVALID;
    const kvfa::DecodeCache cache = k_scale ? kvfa::DecodeCache::kFp8 : kvfa::DecodeCache::kBf16;
    hipError_t e = kvfa::launch_decode_paged(q, k_cache, v_cache, page_table, seq_lens, o, lse,
                                             num_seqs, H, Hkv, d, num_pages, max_pages_per_seq,
                                             max_seq_len, scale, workspace, stream, cache,
                                             k_scale, v_scale);
    return hip_status(e, "decode_checked");
}
}  // namespace

extern "C" {

int fa_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* page_table, const int32_t* seq_lens, int page_size, void* o,
                 float* lse, int B, int H, int Hkv, int Nq, int d, int num_pages,
                 int max_pages_per_seq, int max_seq_len, int causal, float scale,
                 hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !o) return FA_ERR_INVALID;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
        !aligned(page_table, 4) || !aligned(seq_lens, 4))
        return FA_ERR_INVALID;
    if (lse && !aligned(lse, 4)) return FA_ERR_INVALID;
    if (B < 1 || H < 1 || Hkv < 1 || Nq < 1 || num_pages < 1 || max_pages_per_seq < 1)
        return FA_ERR_INVALID;
    if (H % Hkv != 0) return FA_ERR_INVALID;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID;
    if (page_size != 16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
    if (max_seq_len < Nq || (long long)max_pages_per_seq * page_size < max_seq_len)
        return FA_ERR_INVALID;
    if ((unsigned long long)Nq * d * 2 >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
    const unsigned long long n_wg = (unsigned long long)((Nq + 127) / 128) * B * H;
    if (n_wg >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
    hipError_t e = kvfa::launch_fwd_bf16_paged(q, k_cache, v_cache, page_table, seq_lens, o, lse,
                                               B, H, Hkv, Nq, d, num_pages, max_pages_per_seq,
                                               max_seq_len, causal != 0, scale,
                                               stream);
    return hip_status(e, "fa_fwd_paged");
}

int fa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                 const int32_t* page_table, const int32_t* start_pos, int page_size,
                 int num_seqs, int n_new, int Hkv, int d, int num_pages,
                 int max_pages_per_seq, hipStream_t stream) {
    if (!k_new || !v_new || !k_cache || !v_cache || !page_table || !start_pos)
        return FA_ERR_INVALID;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 16) || !aligned(page_table, 4) || !aligned(start_pos, 4))
        return FA_ERR_INVALID;
    if (num_seqs < 1 || n_new < 1 || Hkv < 1 || num_pages < 1 || max_pages_per_seq < 1)
        return FA_ERR_INVALID;
    if (page_size != 16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
    hipError_t e = kvfa::launch_kv_append(k_new, v_new, k_cache, v_cache, page_table, start_pos,
                                          num_seqs, n_new, Hkv, d, num_pages, max_pages_per_seq,
                                          stream);
    return hip_status(e, "fa_kv_append");
}

size_t fa_bwd_workspace_size(int B, int H, int Nq) {
    if (B < 1 || H < 1 || Nq < 1) return 0;
    return kvfa::bwd_workspace_bytes(B, H, Nq);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Nq, int Nk,
           int d, int causal, float scale, void* workspace, size_t workspace_bytes,
           hipStream_t stream) {
    int st = check_prefill(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, causal, scale, 2);
    if (st != FA_OK) return st;
    if (!lse || !dout || !dq || !dk || !dv || !workspace) return FA_ERR_INVALID;
    if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        !aligned(workspace, 4))
        return FA_ERR_INVALID;
    if (workspace_bytes < kvfa::bwd_workspace_bytes(B, H, Nq)) return FA_ERR_INVALID;
    const unsigned long long n_q = (unsigned long long)((Nq + 127) / 128) * B * H;
    const unsigned long long n_k = (unsigned long long)((Nk + 127) / 128) * B * Hkv;
    if (n_q >= (1ull << 31) || n_k >= (1ull << 31)) return FA_ERR_UNSUPPORTED;
    hipError_t e = kvfa::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, B, H, Hkv, Nq, Nk, d,
                                         causal != 0, scale, workspace,
                                         stream);
    return hip_status(e, "fa_bwd");
}

int fa_decode_paged_fp8(const void* q, const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale,
                        const int32_t* page_table, const int32_t* seq_lens, int page_size,
                        void* o, float* lse, int num_seqs, int H, int Hkv, int d,
                        int num_pages, int max_pages_per_seq, int max_seq_len, float scale,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4))
        return FA_ERR_INVALID;
    return decode_checked(q, k_cache, v_cache, page_table, seq_lens, page_size, o, lse, num_seqs,
                          H, Hkv, d, num_pages, max_pages_per_seq, max_seq_len, scale, workspace,
                          workspace_bytes, stream, k_scale, v_scale);
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_SCRATCH:
            return "FA_ERR_SCRATCH: the call needs more workspace than the static scratch of "
                   "fa_decode_paged_noalloc (FA_NOALLOC_SCRATCH_BYTES)";
        case FA_ERR_INVALID: return "FA_ERR_INVALID: an argument is out of its documented range";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: valid request not implemented";
        case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported a launch error";
        default: return "unknown fa_status";
    }
}

}  // extern "C"

// ---- fa_decode_paged_noalloc: the decode workspace in a static device array ----------
// `scratch` exists once per GPU the library runs on (the code object's globals are
// placed on each device when the library's kernels load there) and is kept until the
// process ends. In host code its name is only a stand-in: the device address is looked
// up once per device with hipGetSymbolAddress, with that device current, and that
// address is what the kernels receive. Every call on a device shares the device's
// array, so calls that overlap on one GPU (different streams, or threads) race.
namespace {
__device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];  // device address of `scratch`, per device id

// Device address of the current device's `scratch` (looked up on its first use there).
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "fa_decode_paged_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "fa_decode_paged_noalloc: hipGetSymbolAddress");
        if (p == nullptr) return FA_ERR_HIP;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return FA_OK;
}
}  // namespace

extern "C" int fa_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* page_table, const int32_t* seq_lens,
                                       int page_size, void* o, float* lse, int num_seqs, int H,
                                       int Hkv, int d, int num_pages, int max_pages_per_seq,
                                       int max_seq_len, float scale, hipStream_t stream) {
    const int st = decode_args_status(q, k_cache, v_cache, page_table, seq_lens, page_size, o,
                                      lse, num_seqs, H, Hkv, d, num_pages, max_pages_per_seq,
                                      max_seq_len, scale);
    if (st != FA_OK) return st;
    const size_t need = kvfa::decode_workspace_bytes(num_seqs, H, d, max_seq_len);
    if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    void* ws = nullptr;
    const int sst = scratch_address(&ws);
    if (sst != FA_OK) return sst;
    // Nothing in the workspace has to start at zero: each word a decode call reads was
    // written earlier in the same call (slot counts, partial results, the range plan).
    hipError_t e = kvfa::launch_decode_paged(q, k_cache, v_cache, page_table, seq_lens, o, lse,
                                             num_seqs, H, Hkv, d, num_pages, max_pages_per_seq,
                                             max_seq_len, scale, ws, stream,
                                             kvfa::DecodeCache::kBf16, nullptr, nullptr);
    return hip_status(e, "fa_decode_paged_noalloc");
}
