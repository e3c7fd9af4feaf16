// Host-side launchers shared between the ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/hcsa.h"

namespace hcsa {

// Byte counts rounded up to the 256-byte alignment of workspace parts.
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// ---- compress.hip
hipError_t launch_compress(const void* x, int x_dtype, int64_t x_bstride, int B, int T, int D,
                           const float* omega, int ratio, void* y, int y_dtype,
                           int64_t y_bstride, uint8_t* ys, int64_t ys_bstride,
                           hipStream_t s);
hipError_t launch_compress_batched(const struct hcsa_pool_job* jobs, int n, int B,
                                   const int32_t* block_table, int64_t table_stride, int64_t raw_ring,
                                   hipStream_t s);
hipError_t launch_mxfp4_quantize(const void* x, int x_dtype, int64_t rows, int D,
                                 uint8_t* packed, uint8_t* scales, hipStream_t s);

// ---- topk.hip
struct TopkPlan {
  int rows, N, k, key_bits, nseg;
  bool rows_path;                               // one block per row, no workspace
  size_t floor_off, cnt_off, cand_off, total_bytes;
};
TopkPlan plan_topk(int score_dtype, int rows, int N, int k);
bool topk_plan_ok(const TopkPlan& plan);        // the row length is within the selector's range
hipError_t launch_topk(const TopkPlan& plan, const void* scores, int score_dtype,
                       int64_t row_stride, int Nq, int ratio, int64_t pos0,
                       const int64_t* seq_pos, int32_t* idx, void* ws, hipStream_t s);
// The segment path's device view and workspace of a plan (the decode step runs the extract
// launch itself and the per-row resolve inside its own launch), and the extract launch.
namespace segsel {
struct TopkDev;
struct SegWs;
}
void seg_select_view(const TopkPlan& plan, const void* scores, int64_t row_stride, int Nq,
                     int ratio, int64_t pos0, const int64_t* seq_pos, int32_t* idx, void* ws,
                     segsel::TopkDev* P, segsel::SegWs* S, int* vec);
hipError_t launch_seg_extract(const segsel::TopkDev& P, const segsel::SegWs& S, int vec,
                              int key_bits, int rows, hipStream_t s);

// ---- indexer.hip
hipError_t launch_index_scores(const void* q, int q_dtype, const float* w, const void* kx,
                               int k_dtype, int64_t k_bstride, const uint8_t* ks,
                               int64_t ks_bstride, int B, int Nq, int H_I, int d_I, int N,
                               int ratio, int64_t pos0, const int64_t* seq_pos,
                               const int32_t* block_table, int64_t table_stride,
                               int score_dtype, void* scores, hipStream_t s);

void time_next_indexer(hipEvent_t start, hipEvent_t stop);

// Indexer + top-k of MXFP4 keys without the score array (few long rows, bf16 scores): a
// floor per row from scored samples, the scan's per-chunk candidate lists, the exact
// threshold among them (rows with too few or too many candidates rescanned and selected
// over the whole row).  Same result as launch_index_scores + launch_topk.  With pooling
// jobs (validated, the blocks completed by the query tokens), the pooling runs in the
// floors' launch and the floors sample only entries completed before the query tokens.
bool mx_topk_fused_ok(int rows, int N, int score_dtype);
size_t mx_topk_workspace_bytes(int rows, int N);
hipError_t launch_mxfp4_index_topk(const void* q, int q_dtype, const float* w,
                                   const uint8_t* kx, int64_t k_bstride, const uint8_t* ks,
                                   int64_t ks_bstride, int B, int Nq, int H_I, int d_I, int N,
                                   int ratio, int64_t pos0, const int64_t* seq_pos,
                                   const int32_t* block_table, int64_t table_stride, int k,
                                   int32_t* idx, bool fp8, void* ws, hipStream_t s,
                                   const struct hcsa_pool_job* pool_jobs = nullptr,
                                   int n_pool_jobs = 0, int64_t raw_ring = 0);

// ---- attention.hip
struct AttnArgs {
  const void* q;
  const void* kc;      // compressed K (CSA) or HCA K
  const void* vc;
  int64_t c_bstride;
  int N;
  int ratio;
  const int32_t* idx;  // CSA only (nullptr for HCA)
  int k;
  const void* k_raw;
  const void* v_raw;
  int64_t raw_bstride;
  int64_t T_raw, raw_pos0;
  int n_win;
  int64_t pos0;
  const int64_t* seq_pos;  // [B] or null: query i of sequence b at seq_pos[b] + i
  const int32_t* block_table;   // paged caches [B][table_stride], or null (contiguous)
  int64_t table_stride;
  int64_t raw_ring;        // 0, or raw tokens in a ring of raw_ring rows (position t at t & (raw_ring-1))
  int kv_dtype, B, Nq, H, d;
  float scale;
  float* out;
  float* lse;
};
struct AttnPlan {
  int rows, max_len, chunk, splits;
  bool mfma, tiled, hca_decode;
  size_t part_bytes, total_bytes;
};
// Backward of the attention: the forward's arguments (a) plus these.
struct AttnBwdArgs {
  const float* out;     // forward output [rows][H][d]
  const float* lse;     // forward log-sum-exp [rows][H]
  const float* dout;    // [rows][H][d]
  const float* dlse;    // [rows][H] or null
  float* dq;            // [rows][H][d], written
  float* dkc;           // [B][N][d] F32, accumulated (HCA: the entries)
  float* dvc;
  int64_t dc_bstride;
  float* dkr;           // [B][T_raw][d] F32, accumulated (CSA window rows)
  float* dvr;
  int64_t dr_bstride;
  void* ws;             // bwd_workspace_bytes(a) bytes (or null)
};
// Backward with many query tokens (bf16 16 x 128): the keys shared by consecutive tokens
// (HCA entries, CSA window rows) get their gradients key-major; the per-(token, head) terms
// of the query-major pass reach that kernel through the workspace.
bool bwd_key_major(const AttnArgs& a);
size_t bwd_workspace_bytes(const AttnArgs& a);
// register tiling of the backward kernel: heads rounded up to 4, 16, 32 or 64 and channels
// per lane (d / 64 rounded up to 1, 2 or 4); supported when heads * channels <= 64
inline int bwd_heads(int H) { return H <= 4 ? 4 : H <= 16 ? 16 : H <= 32 ? 32 : H <= 64 ? 64 : 0; }
inline int bwd_cpl(int d) { return d <= 64 ? 1 : d <= 128 ? 2 : d <= 256 ? 4 : 0; }
bool attn_bwd_shape_supported(int H, int d);
hipError_t launch_attention_bwd(bool csa, const AttnArgs& a, const AttnBwdArgs& g, hipStream_t s);
size_t compress_bwd_workspace_bytes(int B, int T, int ratio);
hipError_t launch_compress_bwd(const void* x, int x_dtype, int64_t x_bstride, int B, int T,
                               int D, const float* omega, int ratio, const float* dy,
                               int64_t dy_bstride, float* dx, int64_t dx_bstride,
                               float* domega, void* ws, hipStream_t s);
AttnPlan plan_attention(bool csa, int kv_dtype, int B, int Nq, int H, int d, int max_len);
void set_attn_splits(int splits);   // 0: automatic (this thread's later plans)
// Sets the calling thread's error message (hcsa_last_error) and returns `code`.
int abi_fail(int code, const char* fmt, ...);
hipError_t launch_attention(bool csa, const AttnArgs& a, const AttnPlan& plan, void* ws,
                            hipStream_t s);
// CSA and HCA attention of the same query tokens: one launch for both (plus one merge) on
// the decode fast path, else the two calls in turn; workspace = align256(pc.total_bytes) +
// ph.total_bytes.
bool csa_hca_fused(const AttnPlan& pc, const AttnPlan& ph);
hipError_t launch_csa_hca(const AttnArgs& c, const AttnPlan& pc, const AttnArgs& h,
                          const AttnPlan& ph, void* ws, hipStream_t s);

// ---- decode.hip
// One decode step (pooling of the completed blocks, MXFP4 indexer + top-k without a score
// array, CSA and HCA attention) in four launches with the same results as
// hcsa_csa_pool_index_topk followed by hcsa_csa_hca_attn.
struct DecodeStepArgs {
  const struct hcsa_pool_job* jobs;
  int n_jobs;
  const void* q_idx;
  int q_dtype;
  const float* w_idx;
  const uint8_t* k_idx;
  int k_dtype;
  int64_t k_bstride;
  const uint8_t* k_scales;
  int64_t ks_bstride;
  int H_I, d_I, N, score_dtype;
  int32_t* idx;                 // [B*Nq][k] selection
  const int32_t* block_table;
  int64_t raw_ring;
  const int64_t* seq_pos;
  AttnArgs c, h;                // CSA (k, N, ratio, window) and HCA attention
  int B, Nq;
};
// the four-launch form applies (else the two calls run in turn)
bool decode_step_fast(const DecodeStepArgs& a, const AttnPlan& pc, const AttnPlan& ph,
                      bool fused_selection);
// attention splits of the four-launch form
AttnPlan plan_step_csa(int B, int Nq, int H, int d, int k, int n_win);
AttnPlan plan_step_hca(int B, int Nq, int H, int d, int N_h);
// workspace: [selection state (mx_topk_layout)][sync words at sync_off][attention partials
// at attn_off: CSA, then HCA at align256(pc.total_bytes)]
size_t decode_step_sync_bytes(int rows);
hipError_t launch_decode_step(const DecodeStepArgs& a, const AttnPlan& pc, const AttnPlan& ph,
                              void* ws, size_t sync_off, size_t attn_off, hipStream_t s);
// bf16 or fp32 indexer keys at decode (few long rows): the score-array form (pooling, key
// scan writing scores, segment extract, resolve + CSA beside the HCA splits, merge); its
// selection state is laid out as the selector's own call lays it out, at the workspace start
bool decode_step_scores_ok(const DecodeStepArgs& a, const AttnPlan& pc, const AttnPlan& ph);
hipError_t launch_decode_step_scores(const DecodeStepArgs& a, const AttnPlan& pc,
                                     const AttnPlan& ph, void* ws, size_t sync_off,
                                     size_t attn_off, hipStream_t s);

}  // namespace hcsa
