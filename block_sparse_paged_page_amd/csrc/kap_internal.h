// Internal host-side declarations shared by the libkap HIP sources.
#pragma once

#include "kap_device.h"

namespace kap {

// ---------------------------------------------------------------- host side
void set_error(const char* fmt, ...);
kap_status fail(kap_status s, const char* fmt, ...);
kap_status check_launch(const char* what);
int resident_blocks(const void* kernel, int block_threads);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace carving for the attention calls (decode and verify share it).
struct AttnWorkspace {
  int32_t* n_items;     // [1]
  int32_t* row_off;     // [B*Hkv + 1] first work item of each (b, g)
  float2* part_ml;      // [max_items][R] (reference max in log2 units, sum)
  float* part_o;        // [max_items][R][D] fp32 (bf16, normalized, for the MFMA kernel)
  int32_t max_items;
  size_t bytes;
};
AttnWorkspace carve_attn_workspace(void* base, int32_t B, int32_t q_len, int32_t Hq,
                                   int32_t Hkv, int32_t D);

struct AttnCall {
  const void* q;
  kap_dtype dtype;
  const int32_t* positions;
  int32_t q_len;
  float theta, scale;
  const void* k;
  const void* v;
  int32_t Hkv, D;
  const int32_t* table;
  const int32_t* logical;  // logical page per table entry, or null (entry j is page j)
  int32_t width, G;
  const int32_t* lens;
  int32_t B, Hq;
  void* out;
  float* lse;
  AttnWorkspace ws;
  hipStream_t stream;
};
kap_status launch_attention(const AttnCall& c);

kap_status launch_score(const void* q, kap_dtype q_dt, const int32_t* pos, float theta,
                        const void* summ, kap_dtype s_dt, const int32_t* bt, int32_t max_pages,
                        const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                        float* scores, hipStream_t stream);
// All KV heads per block plus the head-pooled key (scores may be null); Hkv <= 16.
kap_status launch_score_pool(const void* q, kap_dtype q_dt, const int32_t* pos, float theta,
                             const void* summ, kap_dtype s_dt, const int32_t* bt,
                             int32_t max_pages, const int32_t* seq_lens, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t D, float* scores, float* pooled,
                             hipStream_t stream);
kap_status launch_select(const float* scores, int32_t B, int32_t Hkv, int32_t max_pages,
                         const int32_t* seq_lens, int32_t per_head, const int32_t* anchor,
                         const int32_t* recent, const int32_t* k_mid, int32_t capacity,
                         int32_t* sel, int32_t* cnt, hipStream_t stream,
                         const int32_t* bt = nullptr, const int32_t* pos = nullptr,
                         int32_t q_new = 0, int32_t* cbt = nullptr, int32_t* clen = nullptr,
                         int64_t* slot = nullptr);
kap_status launch_compact(const int32_t* sel, const int32_t* cnt, int32_t B, int32_t G,
                          int32_t cap, const int32_t* bt, int32_t max_pages,
                          const int32_t* seq_lens, const int32_t* pos, int32_t q_new,
                          int32_t* cbt, int32_t* clog, int32_t* clen, int64_t* slot,
                          hipStream_t stream);
// first_pos == nullptr: every logical page; else only the pages holding
// tokens first_pos[b] .. first_pos[b] + q_new - 1.
kap_status launch_summary(const void* k, kap_dtype kv_dt, int32_t Hkv, int32_t D,
                          const int32_t* bt, int32_t max_pages, const int32_t* seq_lens,
                          const int32_t* first_pos, int32_t q_new, int32_t B, void* summ,
                          kap_dtype s_dt, hipStream_t stream);
kap_status launch_materialize(const void* k, const void* v, kap_dtype dt, int32_t Hkv, int32_t D,
                              const int32_t* cbt, int32_t B, int32_t G, int32_t cap, void* kws,
                              void* vws, int32_t* ws_table, hipStream_t stream);
kap_status launch_append(const void* k_new, const void* v_new, kap_dtype dt, const int64_t* slot,
                         int32_t B, int32_t q_new, int32_t Hkv, int32_t D, int64_t num_slots,
                         void* k, void* v, hipStream_t stream);
int proxy_splits(int d_model);
kap_status launch_proxy_pack(const uint16_t* wq, uint16_t* wp, int32_t dm, int32_t n_out,
                             hipStream_t stream);
kap_status launch_proxy_packed(const uint16_t* hidden, const uint16_t* wp, int32_t B, int32_t dm,
                               int32_t n_out, float* q_out, hipStream_t stream);
kap_status launch_diag_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);
kap_status launch_proxy(const uint16_t* hidden, const uint16_t* wq, int32_t B, int32_t dm,
                        int32_t n_out, float* q_out, float* partial, int32_t splits,
                        hipStream_t stream);

}  // namespace kap
