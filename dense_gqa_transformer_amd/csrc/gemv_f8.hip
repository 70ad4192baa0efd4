// GEMV instantiations for fp8 (e4m3) weight codes, in a translation unit of
// their own: Q/K/V, gate/up and the head quantize their normalised activation
// rows in the prologue (one or up to four rows per workgroup); the output and
// down projections (residual epilogue) are weight-only.
#include "gemv_impl.h"

namespace fsk {

hipError_t gemv_f8(int epi, GemvParams p, hipStream_t s) {
  if (p.K % 16 != 0 || p.wscale == nullptr) return hipErrorInvalidValue;
  if (epi != EPI_RESID && (!p.aquant || p.M > 4)) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_STORE: return dispatch_mb<f8, EPI_STORE>(p, s);
    case EPI_RESID: return dispatch_mb<f8, EPI_RESID>(p, s);
    case EPI_SWIGLU: return dispatch_mb<f8, EPI_SWIGLU>(p, s);
    case EPI_LOGITS: return dispatch_mb<f8, EPI_LOGITS>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fsk
