// Launch interface of the linear branch's backward (linear_bwd.hip), used
// by the C ABI implementation.
#pragma once

#include "hwa_internal.h"

namespace hwa {

// Backward of the linear branch: device pointers of one call. Inputs as for
// hybrid_attn_fwd; d_o = dL/dy; the rest is workspace (fp32 unless noted):
//   A, Bm, M      [B*H, F, d, d]   statistics, inverses; A and Bm then hold dA, dB
//   Pst, Qst      [B*H, F+1, d, d] P_{s-1} and Q_s of every s; E their row
//                 exponents (int32 [2, B*H, F+1, d])
//   dSt           [B*H, F, d, d]   dS_t of every frame, later dX of the prefix
//                 adjoint (dXP aliases it); dXQ likewise for the suffix
//   dbank         [2, B*H, nch+1, d, d], lam0 [2, B*H, d, d]
//   gab           [2, B*H, F, d] da_t, db_t;  dal, dwpart [B*H, F, d]
//   dkc, dvc      [B*H, N, d]      gradients before the convs
//   cpart         [B*H, F, d, 8]   per-frame tap gradients (k, then v)
struct LinBwdArgs {
  const void *q, *k, *v, *gate, *d_o;
  const float *beta, *alpha, *text_state, *conv_k, *conv_v, *rms_w;
  int rule;
  int acc;  // add dq, dk, dv to the buffers' contents
  float c, text_scale, eps;
  void *dq, *dk, *dv, *dgate;
  float *dbeta, *dalpha, *dtext, *dconv_k, *dconv_v, *drms;
  float *A, *Bm, *M, *Pst, *Qst, *dSt, *dXP, *dXQ, *dbank, *lam0, *gab, *dal, *dwpart;
  float *dkc, *dvc, *cpart;
  int32_t* E;
};

// stage 0: recompute (statistics, inverses, every frame's states); 1: readout;
// 2: gather, adjoint scans, frame gradients; 3: statistics and features;
// 4: convs, dalpha and the parameter sums.
hipError_t launch_linear_bwd(const Geom& g, int dtype, int stage, const LinBwdArgs& a,
                             hipStream_t st);

}  // namespace hwa
