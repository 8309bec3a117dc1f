// Host-side launchers of the attention kernels. Arguments are already validated by
// the C ABI layer (api.hip); each launcher only enqueues work on `stream` and returns
// the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvfa {

hipError_t launch_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse,
                           int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                           hipStream_t stream);

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                           hipStream_t stream);

// The key-split prefill kernel (64-row work-groups whose key range runs in four parts);
// launch_fwd_bf16 picks it for launches of at most 128 blocks of 256 rows.
hipError_t launch_fwd_bf16_key_split(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int B, int H, int Hkv, int Nq, int Nk, int d,
                                     int causal, float scale, hipStream_t stream);

hipError_t launch_fwd_bf16_two_pass(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int B, int H, int Hkv, int Nq, int Nk, int d,
                                    int causal, float scale, hipStream_t stream);

hipError_t launch_fwd_bf16_window(const void* q, const void* k, const void* v, void* o,
                                  float* lse, int B, int H, int Hkv, int Nq, int Nk, int d,
                                  int window_left, int window_right, float scale,
                                  hipStream_t stream);

hipError_t launch_fwd_bf16_paged(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* page_table, const int32_t* seq_lens, void* o,
                                 float* lse, int B, int H, int Hkv, int Nq, int d, int num_pages,
                                 int max_pages_per_seq, int max_seq_len, int causal, float scale,
                                 hipStream_t stream);

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* page_table, const int32_t* start_pos, int num_seqs,
                            int n_new, int Hkv, int d, int num_pages, int max_pages_per_seq,
                            hipStream_t stream);

// Backward pass: workspace bytes (the rows' D = rowsum(dO * O)) and the launcher.
size_t bwd_workspace_bytes(int B, int H, int Nq);
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                           void* workspace, hipStream_t stream);

// Decode range plan: the fewest cached tokens a split-K work-group's range holds, the
// work-groups per (KV head, head group) the longest possible cache needs, and the
// workspace the plan implies.
// (16-token pages throughout.)
int decode_split_tokens(int num_seqs, int max_seq_len);
int decode_min_work_groups(int num_seqs, int max_seq_len);
size_t decode_workspace_bytes(int num_seqs, int H, int d, int max_seq_len);

// Element type of the paged cache. An e4m3 cache comes with its per-KV-head scales
// (k_scale, v_scale non-null); a bf16 cache has none (both null). The launcher returns
// hipErrorInvalidValue, enqueueing nothing, when the pointers do not match the type.
enum class DecodeCache { kBf16, kFp8 };

hipError_t launch_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* page_table, const int32_t* seq_lens, void* o,
                               float* lse, int num_seqs, int H, int Hkv, int d, int num_pages,
                               int max_pages_per_seq, int max_seq_len, float scale,
                               void* workspace, hipStream_t stream, DecodeCache cache,
                               const float* k_scale, const float* v_scale);

}  // namespace kvfa
