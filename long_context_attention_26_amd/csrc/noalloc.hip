// The decode step without a caller-supplied workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the step's workspace is a fixed scratch array in the library's own device
// memory, one copy per GPU, held until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace {

constexpr size_t kScratchBytes = HCSA_DECODE_STEP_SCRATCH_BYTES;

// Host code sees only a stand-in for this name; kernels get the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// This device's copy of `scratch`, looked up on the first call on the device (with that
// device current) and kept.
int scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hcsa::abi_fail(HCSA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return hcsa::abi_fail(HCSA_EINVAL, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return hcsa::abi_fail(HCSA_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                            hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return HCSA_OK;
}

}  // namespace

extern "C" int hcsa_decode_step_noalloc(
    const hcsa_pool_job* jobs, int n_jobs, const void* q_idx, int q_dtype, const float* w_idx,
    const void* k_idx, int k_dtype, int64_t k_bstride, const uint8_t* k_scales,
    int64_t ks_bstride, int H_I, int d_I, int score_dtype, int32_t* topk_idx, const void* q,
    const void* kc, const void* vc, int64_t c_bstride, int N, int k, const void* k_raw,
    const void* v_raw, int64_t raw_bstride, int64_t T_raw, int64_t raw_pos0, int n_win,
    int ratio, const void* kh, const void* vh, int64_t h_bstride, int N_h, int ratio_h,
    int64_t pos0, const int64_t* seq_pos, const hcsa_pages* pages, int kv_dtype, int B, int Nq,
    int H, int d, float scale, float* out_c, float* lse_c, float* out_h, float* lse_h,
    hcsa_stream stream) {
  const size_t need =
      hcsa_decode_step_workspace_size(B, Nq, N, k, score_dtype, H, d, n_win, N_h);
  if (need > kScratchBytes)
    return hcsa::abi_fail(HCSA_EWORKSPACE,
                          "hcsa_decode_step_noalloc: this step needs %zu bytes of workspace, "
                          "the fixed scratch holds %zu (use hcsa_decode_step)",
                          need, kScratchBytes);
  void* ws = nullptr;
  if (const int rc = scratch_for_current_device(&ws)) return rc;
  return hcsa_decode_step(jobs, n_jobs, q_idx, q_dtype, w_idx, k_idx, k_dtype, k_bstride,
                          k_scales, ks_bstride, H_I, d_I, score_dtype, topk_idx, q, kc, vc,
                          c_bstride, N, k, k_raw, v_raw, raw_bstride, T_raw, raw_pos0, n_win,
                          ratio, kh, vh, h_bstride, N_h, ratio_h, pos0, seq_pos, pages,
                          kv_dtype, B, Nq, H, d, scale, out_c, lse_c, out_h, lse_h, ws,
                          kScratchBytes, stream);
}
