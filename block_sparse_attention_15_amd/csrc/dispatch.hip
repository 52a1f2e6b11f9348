// Kernel selection for the attention forward and backward.
#include "common.h"

namespace pbsa {

hipError_t launch_fwd_simple(const Geo& g, const void* q, const void* k_p, const void* v_p, const int32_t* plen,
                             const void* k_l, const void* v_l, const int32_t* topk, void* o, float* lse,
                             float* blse_p, float* blse_l, hipStream_t s);
bool fwd_mfma_supported(const Geo& g);
size_t fwd_mfma_workspace(const Geo& g);
hipError_t launch_fwd_mfma(const Geo& g, const void* q, const void* k_p, const void* v_p, const int32_t* plen,
                           const void* k_l, const void* v_l, const int32_t* topk, void* o, float* lse, void* ws,
                           float* blse_p, float* blse_l, hipStream_t s);
hipError_t launch_bwd_prep(const Geo& g, const void* o, const void* dout, const float* lse, const int32_t* topk,
                           WsBwd ws, hipStream_t s);
hipError_t launch_bwd_simple(const Geo& g, const void* q, const void* k_p, const void* v_p, const int32_t* plen,
                             const void* k_l, const void* v_l, const int32_t* topk, const float* lse,
                             const void* dout, float* dq, float* dk_p, float* dv_p, float* dk_l, float* dv_l,
                             WsBwd ws, hipStream_t s);

size_t fwd_workspace(const Geo& g) { return fwd_mfma_supported(g) ? fwd_mfma_workspace(g) : 0; }

hipError_t launch_bwd_mfma(const Geo& g, const void* q, const void* k_p, const void* v_p, const int32_t* plen,
                           const void* k_l, const void* v_l, const int32_t* topk, const void* o, const float* lse,
                           const void* dout, float* dq, float* dk_p, float* dv_p, float* dk_l, float* dv_l,
                           WsBwd ws, hipStream_t s);

hipError_t launch_fwd(const Geo& g, const void* q, const void* k_p, const void* v_p, const int32_t* plen,
                      const void* k_l, const void* v_l, const int32_t* topk, void* o, float* lse, void* ws,
                      float* blse_p, float* blse_l, hipStream_t s) {
  if (fwd_mfma_supported(g))
    return launch_fwd_mfma(g, q, k_p, v_p, plen, k_l, v_l, topk, o, lse, ws, blse_p, blse_l, s);
  return launch_fwd_simple(g, q, k_p, v_p, plen, k_l, v_l, topk, o, lse, blse_p, blse_l, s);
}

hipError_t launch_bwd(const Geo& g, const void* q, const void* k_p, const void* v_p, const int32_t* plen,
                      const void* k_l, const void* v_l, const int32_t* topk, const void* o,
                      const float* lse, const void* dout, float* dq, float* dk_p, float* dv_p,
                      float* dk_l, float* dv_l, WsBwd ws, hipStream_t s) {
  if (bwd_mfma_supported(g))  // runs its own preparation, partly on its second stream
    return launch_bwd_mfma(g, q, k_p, v_p, plen, k_l, v_l, topk, o, lse, dout, dq, dk_p, dv_p, dk_l, dv_l, ws, s);
  hipError_t e = launch_bwd_prep(g, o, dout, lse, topk, ws, s);
  if (e != hipSuccess) return e;
  return launch_bwd_simple(g, q, k_p, v_p, plen, k_l, v_l, topk, lse, dout, dq, dk_p, dv_p, dk_l, dv_l, ws, s);
}

}  // namespace pbsa
