// Dual-timescale query summaries (GrowPage Sec. 3.2 Eq. 6; App. E.1 slot pool and first-step
// initialisation). One thread per 4 consecutive elements of a request's H_q * d query.
#include "common.h"

namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void ema_kernel(const void* __restrict__ q, int B, int HD,
                                                  const int32_t* __restrict__ slot_ids,
                                                  const uint8_t* __restrict__ fresh,
                                                  float* __restrict__ qstate, int num_slots,
                                                  float beta_s, float beta_l) {
  const int r = blockIdx.y;
  const int i = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= HD) return;
  const int slot = slot_ids[r];
  if (slot < 0 || slot >= num_slots) return;
  float x[4];
  gp::load_q4<BF16>(q, (size_t)r * HD + i, x);
  gp::ema_update4(qstate + ((size_t)slot * 2 + 0) * HD + i, qstate + ((size_t)slot * 2 + 1) * HD + i,
                  x, fresh[r] != 0, beta_s, beta_l);
}

}  // namespace

extern "C" int gp_update_query_summaries(const void* q, int q_dtype, int B, int H_q, int head_dim,
                                         const int32_t* slot_ids, const uint8_t* fresh,
                                         float* qstate, int num_slots, float beta_s, float beta_l,
                                         void* stream) {
  if (B < 0 || H_q <= 0 || head_dim <= 0 || num_slots <= 0) return GP_ERR_INVALID;
  if (B == 0) return GP_OK;
  if (!q || !slot_ids || !fresh || !qstate) return GP_ERR_INVALID;
  if (q_dtype != GP_F32 && q_dtype != GP_BF16) return GP_ERR_INVALID;
  const int HD = H_q * head_dim;
  if (HD % 4 != 0) return GP_ERR_UNSUPPORTED;
  dim3 grid((HD / 4 + 255) / 256, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q_dtype == GP_BF16)
    hipLaunchKernelGGL(ema_kernel<true>, grid, dim3(256), 0, s, q, B, HD, slot_ids, fresh, qstate,
                       num_slots, beta_s, beta_l);
  else
    hipLaunchKernelGGL(ema_kernel<false>, grid, dim3(256), 0, s, q, B, HD, slot_ids, fresh, qstate,
                       num_slots, beta_s, beta_l);
  GP_CHECK_LAUNCH();
  return GP_OK;
}

extern "C" int gp_version(void) { return GP_VERSION; }

extern "C" const char* gp_status_string(int status) {
  switch (status) {
    case GP_OK: return "ok";
    case GP_ERR_INVALID: return "invalid argument";
    case GP_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case GP_ERR_WORKSPACE: return "workspace missing or too small";
    case GP_ERR_HIP: return "HIP launch failed";
    case GP_ERR_SCRATCH: return "call needs more scratch than the static buffer holds";
    default: return "unknown status";
  }
}
