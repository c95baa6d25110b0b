// Backward of the linear branch (VDN-H3 article, "Step 1" .. "Step 5" and
// "Text state"; the gradients its "Training" section needs). For a loss L
// with upstream gradient G = dL/dy of the branch output y, with the forward's
// notation:
//   q^ = L2(SiLU(q)), k^ = L2(SiLU(conv_k(k))), v^ = conv_v(v)
//   A_f = sum_n beta_n k^_n k^_n^T,  B_f = sum_n beta_n v^_n k^_n^T
//   M_f = (I + cc A_f)^-1, X = S diag(alpha_f) + c1 B_f, R_f(S) = X M_f
//     (vdn_solve: cc = c1 = 1; vdn_scaled: cc = c^2, c1 = c)
//   P_{-1} = Q_F = s0 = text_scale S_text, P_f = R_f(P_{f-1}), Q_f = R_f(Q_{f+1})
//   S_t = P_{lo-1} diag(a_t) + Q_{hi+1} diag(b_t),
//     a_t = prod_{l=lo..t} alpha_l, b_t = prod_{l=t..hi} alpha_l
//   o = S_t q^, z = o / sqrt(mean(o^2) + eps), y = z * w * sigmoid(gate)
// the reverse pass is:
//   readout    dgate, dw, do = r (dz - z mean(dz z)), dq^ = S_t^T do,
//              dS_t = sum_n do_n q^_n^T, dq through L2 and SiLU
//   gather     dP_{lo-1} += dS_t diag(a_t), dQ_{hi+1} += dS_t diag(b_t),
//              da_t = colsum(dS_t * P_{lo-1}), db_t = colsum(dS_t * Q_{hi+1})
//   scans      (adjoint, opposite order) dX = lam M_f^T, lam <- dX diag(alpha_f)
//              (+ the gather's bank gradients); dA_f = -cc P_f^T dX^P - cc
//              Q_f^T dX^Q, dB_f = c1 (dX^P + dX^Q), dalpha_f = colsum(dX^P *
//              P_{f-1} + dX^Q * Q_{f+1}); dS_text = text_scale (lam_P + lam_Q)
//   statistics dk^ = beta (dA + dA^T) k^ + beta dB^T v^, dv^ = beta dB k^,
//              dbeta = k^.(dA k^) + v^.(dB k^), then L2, SiLU and the convs
// All arithmetic is fp32 (bf16 calls: the recomputed scan is the forward's
// split-bf16 MFMA scan). The forward's states are recomputed first with its
// own statistics, inverse and scan kernels (every frame kept: a scan with
// chunk 1 stores one bank slot per frame). Every output element is one fixed
// sum: no atomics, so repeated calls agree bit for bit.

#include "linear_bwd.h"

namespace hwa {

namespace {

// d/dx x sigmoid(x) = s (1 + x (1 - s))
__device__ __forceinline__ float silu_grad(float x) {
  const float s = sigmoid_f(x);
  return s * fmaf(x, 1.0f - s, 1.0f);
}

// Gradient through x^ = u / max(||u||, 1e-12) given dx^, x^, inv = 1 / max(..),
// dot = x^ . dx^ over the vector; a clamped norm passes dx^ * inv straight.
__device__ __forceinline__ float l2_grad(float dxh, float xh, float inv, float dot,
                                         bool clamped) {
  return clamped ? dxh * inv : (dxh - xh * dot) * inv;
}

template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = 1; off < W; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

constexpr int LB_TT = 32;  // readout backward: tokens per tile (8 lanes each)
constexpr int SB_TT = 16;  // statistics backward: tokens per tile (16 lanes each)
constexpr int AJ_R = 8;    // adjoint scan: state rows per workgroup

}  // namespace

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- exponents
// The scan keeps row = stored * 2^e; fold e into the stored rows.
__global__ __launch_bounds__(256) void fold_exp_kernel(float* __restrict__ Pst,
                                                       float* __restrict__ Qst,
                                                       const int32_t* __restrict__ E,
                                                       long long rows, int D) {
  const long long n = rows * D;
  for (long long x = blockIdx.x * 256LL + threadIdx.x; x < 2 * n; x += (long long)gridDim.x * 256) {
    const int dir = x >= n;
    const long long y = x - dir * n;
    const int e = E[dir * rows + y / D];
    if (e != 0) {
      float* p = (dir ? Qst : Pst) + y;
      *p = ldexpf(*p, e);
    }
  }
}

// ---------------------------------------------------------------- readout
// One workgroup per (b, h, frame t): S_t in LDS; tokens 32 at a time, 8 lanes
// per token, lane l owning channels l, l + 8, ...; dS_t accumulates in
// registers, thread (ib, jb) owning rows ib + 16a and columns jb + 16b.
template <typename T, int D>
__global__ __launch_bounds__(256) void lin_readout_bwd_kernel(
    const T* __restrict__ q, const T* __restrict__ gate, const T* __restrict__ gout,
    const float* __restrict__ alpha, const float* __restrict__ Pst,
    const float* __restrict__ Qst, const float* __restrict__ rms_w, float eps,
    T* __restrict__ dq, T* __restrict__ dgate, float* __restrict__ dSt,
    float* __restrict__ dwpart, int F, int S, int chunk, int radius, long long N, int accum) {
  constexpr int LD = D + 1;
  constexpr int TPT = 256 / LB_TT;
  constexpr int CPT = D / TPT;
  constexpr int BS = D / 16;
  __shared__ float st_lds[D * LD];
  __shared__ float qh_lds[LB_TT][D + 4];
  __shared__ float do_lds[LB_TT][D + 4];
  __shared__ float dec[2][D];

  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const int bh = blockIdx.y;
  int lo, hi;
  window_of(t, F, chunk, radius, lo, hi);
  for (int j = tid; j < D; j += 256) {
    const float* al = alpha + (long long)bh * F * D + j;
    float a = 1.0f, b = 1.0f;
    for (int x = lo; x <= t; ++x) a *= al[(long long)x * D];
    for (int x = t; x <= hi; ++x) b *= al[(long long)x * D];
    dec[0][j] = a;
    dec[1][j] = b;
  }
  __syncthreads();
  const float* Pm = Pst + ((long long)bh * (F + 1) + lo) * D * D;      // P_{lo-1}
  const float* Qm = Qst + ((long long)bh * (F + 1) + hi + 1) * D * D;  // Q_{hi+1}
  for (int x = tid; x < D * D; x += 256) {
    const int i = x / D, j = x % D;
    st_lds[i * LD + j] = fmaf(Pm[x], dec[0][j], Qm[x] * dec[1][j]);
  }

  const int tt = tid / TPT, ln = tid % TPT;
  const int ib = tid / 16, jb = tid % 16;
  float wr[CPT], dw[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    wr[c] = rms_w ? rms_w[ln + TPT * c] : 1.0f;
    dw[c] = 0.0f;
  }
  float acc[BS][BS];
#pragma unroll
  for (int a = 0; a < BS; ++a)
#pragma unroll
    for (int b = 0; b < BS; ++b) acc[a][b] = 0.0f;
  const long long base = (long long)bh * N * D;
  __syncthreads();

  for (int s0 = 0; s0 < S; s0 += LB_TT) {
    const int s = s0 + tt;
    const bool valid = s < S;
    const long long row = base + ((long long)t * S + s) * D + ln;
    float qv[CPT], qh[CPT];
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      qv[c] = valid ? ld_io<T>(q, row + TPT * c) : 0.0f;
      qh[c] = silu_f(qv[c]);
      ss = fmaf(qh[c], qh[c], ss);
    }
    ss = group_sum<TPT>(ss);
    const float inv = inv_l2(ss);
    const bool clamped = ss <= 1e-24f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      qh[c] *= inv;
      qh_lds[tt][ln + TPT * c] = qh[c];
    }
    __syncthreads();
    float o[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) o[c] = 0.0f;
    for (int j = 0; j < D; ++j) {
      const float x = qh_lds[tt][j];
#pragma unroll
      for (int c = 0; c < CPT; ++c) o[c] = fmaf(st_lds[(ln + TPT * c) * LD + j], x, o[c]);
    }
    float ms = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) ms = fmaf(o[c], o[c], ms);
    ms = group_sum<TPT>(ms);
    const float r = 1.0f / sqrtf(ms / D + eps);
    float z[CPT], dz[CPT];
    float dzz = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const long long ix = row + TPT * c;
      const float gt = valid ? ld_io<T>(gate, ix) : 0.0f;
      const float go = valid ? ld_io<T>(gout, ix) : 0.0f;
      const float sg = sigmoid_f(gt);
      z[c] = o[c] * r;
      if (valid) st_io<T>(dgate, ix, go * z[c] * wr[c] * sg * (1.0f - sg));
      dw[c] = fmaf(go * sg, z[c], dw[c]);
      dz[c] = go * wr[c] * sg;
      dzz = fmaf(dz[c], z[c], dzz);
    }
    const float mz = group_sum<TPT>(dzz) / D;
#pragma unroll
    for (int c = 0; c < CPT; ++c) do_lds[tt][ln + TPT * c] = r * (dz[c] - z[c] * mz);
    __syncthreads();
    float dqh[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) dqh[c] = 0.0f;
    for (int i = 0; i < D; ++i) {
      const float di = do_lds[tt][i];
#pragma unroll
      for (int c = 0; c < CPT; ++c) dqh[c] = fmaf(st_lds[i * LD + ln + TPT * c], di, dqh[c]);
    }
    float dot = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) dot = fmaf(qh[c], dqh[c], dot);
    dot = group_sum<TPT>(dot);
    if (valid) {
#pragma unroll
      for (int c = 0; c < CPT; ++c)
        st_io<T>(dq, row + TPT * c,
                 l2_grad(dqh[c], qh[c], inv, dot, clamped) * silu_grad(qv[c]) +
                     (accum ? ld_io<T>(dq, row + TPT * c) : 0.0f));
    }
    const int ntok = min(LB_TT, S - s0);
    for (int x = 0; x < ntok; ++x) {
      float dr[BS], qr[BS];
#pragma unroll
      for (int a = 0; a < BS; ++a) {
        dr[a] = do_lds[x][ib + 16 * a];
        qr[a] = qh_lds[x][jb + 16 * a];
      }
#pragma unroll
      for (int a = 0; a < BS; ++a)
#pragma unroll
        for (int b = 0; b < BS; ++b) acc[a][b] = fmaf(dr[a], qr[b], acc[a][b]);
    }
    __syncthreads();
  }
  float* ds = dSt + ((long long)bh * F + t) * D * D;
#pragma unroll
  for (int a = 0; a < BS; ++a)
#pragma unroll
    for (int b = 0; b < BS; ++b) ds[(ib + 16 * a) * D + jb + 16 * b] = acc[a][b];
  // dw partial of this frame: sum over the 32 token slots
#pragma unroll
  for (int c = 0; c < CPT; ++c) qh_lds[tt][ln + TPT * c] = dw[c];
  __syncthreads();
  for (int j = tid; j < D; j += 256) {
    float sum = 0.0f;
    for (int x = 0; x < LB_TT; ++x) sum += qh_lds[x][j];
    dwpart[((long long)bh * F + t) * D + j] = sum;
  }
}

// ---------------------------------------------------------------- gather
// One workgroup per (bank slot m, direction, b*h). Slot m stands for the
// state P_{pos-1} (prefix) or Q_pos (suffix), pos = min(F, m chunk); it sums
// dS_t diag(a_t) (or b_t) over the frames t that gather it and writes
// da_t / db_t (column sums of dS_t times that state) of those frames.
template <int D>
__global__ __launch_bounds__(256) void lin_gather_bwd_kernel(
    const float* __restrict__ dSt, const float* __restrict__ alpha,
    const float* __restrict__ Pst, const float* __restrict__ Qst, float* __restrict__ dbank,
    float* __restrict__ gab, int F, int chunk, int radius, int nch, int BH) {
  constexpr int RG = 256 / D;  // row groups
  constexpr int RPT = D / RG;  // rows per thread
  __shared__ float red[RG][D];
  const int tid = threadIdx.x;
  const int m = blockIdx.x, dir = blockIdx.y, bh = blockIdx.z;
  const int j = tid % D, rg = tid / D;
  const int pos = min(F, m * chunk);
  const float* X = (dir == 0 ? Pst : Qst) + ((long long)bh * (F + 1) + pos) * D * D;
  float xs[RPT], acc[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    xs[k] = X[(rg + RG * k) * D + j];
    acc[k] = 0.0f;
  }
  const float* al = alpha + (long long)bh * F * D + j;
  for (int t = 0; t < F; ++t) {
    int lo, hi;
    window_of(t, F, chunk, radius, lo, hi);
    if ((dir == 0 ? lo : hi + 1) != pos) continue;  // uniform over the workgroup
    float coef = 1.0f;
    const int x0 = dir == 0 ? lo : t, x1 = dir == 0 ? t : hi;
    for (int x = x0; x <= x1; ++x) coef *= al[(long long)x * D];
    const float* ds = dSt + ((long long)bh * F + t) * D * D;
    float part = 0.0f;
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const float v = ds[(rg + RG * k) * D + j];
      acc[k] = fmaf(v, coef, acc[k]);
      part = fmaf(v, xs[k], part);
    }
    red[rg][j] = part;
    __syncthreads();
    if (tid < D) {
      float sum = 0.0f;
#pragma unroll
      for (int g = 0; g < RG; ++g) sum += red[g][tid];
      gab[(((long long)dir * BH + bh) * F + t) * D + tid] = sum;
    }
    __syncthreads();
  }
  float* out = dbank + (((long long)dir * BH + bh) * (nch + 1) + m) * D * D;
#pragma unroll
  for (int k = 0; k < RPT; ++k) out[(rg + RG * k) * D + j] = acc[k];
}

// ---------------------------------------------------------------- adjoint scans
// The adjoint of each scan runs in the opposite frame order. The update
// right-multiplies the state, so adjoint rows are independent as well: a
// workgroup owns 8 rows of one (b*h, direction) chain, M_f staged in LDS.
// Writes dX of every frame and the adjoint of s0.
template <int D>
__global__ __launch_bounds__(256) void lin_adjoint_kernel(
    const float* __restrict__ Mi, const float* __restrict__ alpha,
    const float* __restrict__ dbank, float* __restrict__ dXP, float* __restrict__ dXQ,
    float* __restrict__ lam0, int F, int chunk, int nch, int BH) {
  constexpr int TPR = D / 4;
  __shared__ __attribute__((aligned(16))) float g_lds[D * D];
  __shared__ float x_lds[AJ_R][D];
  const int tid = threadIdx.x;
  const int rb = blockIdx.x, dir = blockIdx.y, bh = blockIdx.z;
  const int r = tid / TPR, j0 = (tid % TPR) * 4;
  const bool active = r < AJ_R;
  const int row = rb * AJ_R + r;
  const float* db = dbank + ((long long)dir * BH + bh) * (nch + 1) * D * D;
  float lam[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  auto inject = [&](int slot) {
    if (!active) return;
    const float4 v = *(const float4*)&db[((long long)slot * D + row) * D + j0];
    lam[0] += v.x;
    lam[1] += v.y;
    lam[2] += v.z;
    lam[3] += v.w;
  };
  inject(dir == 0 ? nch : 0);  // P_{F-1} / Q_0
  float* dX = dir == 0 ? dXP : dXQ;
  // M_f of the next step is fetched into registers while this step computes
  constexpr int NV = D * D / 4;  // 16-byte pieces of one M_f
  constexpr int MV = NV >= 256 ? NV / 256 : 1;
  f32x4_t mreg[MV];
  {
    const f32x4_t* src = (const f32x4_t*)&Mi[((long long)bh * F + (dir == 0 ? F - 1 : 0)) * D * D];
#pragma unroll
    for (int u = 0; u < MV; ++u) mreg[u] = (NV >= 256 || tid < NV) ? src[tid + 256 * u] : f32x4_t{};
  }
  for (int i = 0; i < F; ++i) {
    const int f = dir == 0 ? F - 1 - i : i;
    const long long mo = ((long long)bh * F + f) * D * D;
#pragma unroll
    for (int u = 0; u < MV; ++u)
      if (NV >= 256 || tid < NV) *(f32x4_t*)&g_lds[(tid + 256 * u) * 4] = mreg[u];
    if (active) {
#pragma unroll
      for (int u = 0; u < 4; ++u) x_lds[r][j0 + u] = lam[u];
    }
    __syncthreads();
    if (i + 1 < F) {
      const f32x4_t* src =
          (const f32x4_t*)&Mi[((long long)bh * F + (dir == 0 ? f - 1 : f + 1)) * D * D];
#pragma unroll
      for (int u = 0; u < MV; ++u)
        mreg[u] = (NV >= 256 || tid < NV) ? src[tid + 256 * u] : f32x4_t{};
    }
    if (active) {
      float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      // dX = lam M_f^T = lam M_f (M_f is the inverse of a symmetric matrix)
#pragma unroll 8
      for (int kk = 0; kk < D; ++kk) {
        const float xv = x_lds[r][kk];
        const float4 gv = *(const float4*)&g_lds[kk * D + j0];
        acc[0] = fmaf(xv, gv.x, acc[0]);
        acc[1] = fmaf(xv, gv.y, acc[1]);
        acc[2] = fmaf(xv, gv.z, acc[2]);
        acc[3] = fmaf(xv, gv.w, acc[3]);
      }
      *(float4*)&dX[mo + (long long)row * D + j0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      const float4 a4 = *(const float4*)&alpha[((long long)bh * F + f) * D + j0];
      lam[0] = acc[0] * a4.x;
      lam[1] = acc[1] * a4.y;
      lam[2] = acc[2] * a4.z;
      lam[3] = acc[3] * a4.w;
    }
    if (dir == 0) {
      if (f % chunk == 0) inject(f / chunk);  // P_{f-1} is bank slot f / chunk
    } else {
      if ((f + 1) % chunk == 0 || f + 1 == F) inject((f + chunk) / chunk);  // Q_{f+1}
    }
    __syncthreads();
  }
  if (active)
    *(float4*)&lam0[(((long long)dir * BH + bh) * D + row) * D + j0] =
        make_float4(lam[0], lam[1], lam[2], lam[3]);
}

// ---------------------------------------------------------------- frame gradients
// One workgroup per (frame, b*h): dB_f, dA_f (into the buffers A_f, B_f had)
// and the scans' part of dalpha_f.
// vdn rules (S_f = X_f M_f, M_f = (I + cc A_f)^-1, X_f = S_{f-1} D_f + c1 B_f):
//   dA_f = -cc (P_f^T dX^P_f + Q_f^T dX^Q_f), dB_f = c1 (dX^P_f + dX^Q_f).
// SANA (S_f = X_f M_f + c2 B_f, M_f = I - cc A_f, X_f = S_{f-1} D_f): with
// lam_f = dL/dS_f, dA_f = -cc D_f (P_{f-1}^T lam^P_f + Q_{f+1}^T lam^Q_f) and
// dB_f = c2 (lam^P_f + lam^Q_f). lam_f is rebuilt as the adjoint scan formed
// it: lam^P_f = dX^P_{f+1} D_{f+1} (+ the bank gradient when P_f is a bank
// slot; lam^P_{F-1} is slot nch's alone), lam^Q_f = dX^Q_{f-1} D_{f-1} (+ the
// bank gradient when Q_f is a slot; lam^Q_0 is slot 0's alone).
// Both: dalpha_f = colsum(dX^P_f * P_{f-1} + dX^Q_f * Q_{f+1}).
template <int D, bool SANA>
__global__ __launch_bounds__(256) void lin_frame_grad_kernel(
    const float* __restrict__ Pst, const float* __restrict__ Qst,
    const float* __restrict__ dXP, const float* __restrict__ dXQ, float cc, float cb,
    const float* __restrict__ alpha, const float* __restrict__ dbank, int chunk, int nch,
    int BH, float* __restrict__ dA, float* __restrict__ dB, float* __restrict__ dal, int F) {
  constexpr int BS = D / 16;
  constexpr int KR = 16;
  constexpr int RG = 256 / D, RPT = D / RG;
  __shared__ float sp[KR][D + 4], sxp[KR][D + 4], sq[KR][D + 4], sxq[KR][D + 4];
  __shared__ float red[RG][D];
  const int tid = threadIdx.x;
  const int f = blockIdx.x, bh = blockIdx.y;
  const long long fo = ((long long)bh * F + f) * D * D;
  const long long so = (long long)bh * (F + 1) * D * D;
  const float* P0 = Pst + so + (long long)f * D * D;        // P_{f-1}
  const float* P1 = Pst + so + (long long)(f + 1) * D * D;  // P_f
  const float* Q0 = Qst + so + (long long)f * D * D;        // Q_f
  const float* Q1 = Qst + so + (long long)(f + 1) * D * D;  // Q_{f+1}
  const float* xp = dXP + fo;
  const float* xq = dXQ + fo;
  // SANA: lam^P_f and lam^Q_f at element ix = row * D + col
  const float* xpn = dXP + fo + (long long)D * D;  // dX^P_{f+1} (read when f + 1 < F)
  const float* xqp = dXQ + fo - (long long)D * D;  // dX^Q_{f-1} (read when f >= 1)
  const float* apn = alpha + ((long long)bh * F + f + 1) * D;
  const float* aqp = alpha + ((long long)bh * F + f - 1) * D;
  const int slot_p = f == F - 1 ? nch : ((f + 1) % chunk == 0 ? (f + 1) / chunk : -1);
  const int slot_q = f == 0 ? 0 : (f % chunk == 0 ? f / chunk : -1);
  const float* bp = dbank + ((long long)bh * (nch + 1) + slot_p) * D * D;
  const float* bq = dbank + (((long long)BH + bh) * (nch + 1) + slot_q) * D * D;
  auto lam_p = [&](long long ix, int col) {
    float x = f + 1 < F ? xpn[ix] * apn[col] : 0.0f;
    if (slot_p >= 0) x += bp[ix];
    return x;
  };
  auto lam_q = [&](long long ix, int col) {
    float x = f >= 1 ? xqp[ix] * aqp[col] : 0.0f;
    if (slot_q >= 0) x += bq[ix];
    return x;
  };
  {
    const int j = tid % D, rg = tid / D;
    float part = 0.0f;
#pragma unroll 4
    for (int k = 0; k < RPT; ++k) {
      const long long ix = (long long)(rg + RG * k) * D + j;
      const float a = xp[ix], b = xq[ix];
      if constexpr (SANA)
        dB[fo + ix] = cb * (lam_p(ix, j) + lam_q(ix, j));
      else
        dB[fo + ix] = cb * (a + b);
      part = fmaf(a, P0[ix], part);
      part = fmaf(b, Q1[ix], part);
    }
    red[rg][j] = part;
    __syncthreads();
    if (tid < D) {
      float sum = 0.0f;
#pragma unroll
      for (int g = 0; g < RG; ++g) sum += red[g][tid];
      dal[((long long)bh * F + f) * D + tid] = sum;
    }
  }
  const int ib = tid / 16, jb = tid % 16;
  float acc[BS][BS];
#pragma unroll
  for (int a = 0; a < BS; ++a)
#pragma unroll
    for (int b = 0; b < BS; ++b) acc[a][b] = 0.0f;
  for (int i0 = 0; i0 < D; i0 += KR) {
    __syncthreads();
    for (int x = tid; x < KR * D; x += 256) {
      const int rr = x / D, col = x % D;
      const long long ix = (long long)(i0 + rr) * D + col;
      if constexpr (SANA) {
        sp[rr][col] = P0[ix];
        sxp[rr][col] = lam_p(ix, col);
        sq[rr][col] = Q1[ix];
        sxq[rr][col] = lam_q(ix, col);
      } else {
        sp[rr][col] = P1[ix];
        sxp[rr][col] = xp[ix];
        sq[rr][col] = Q0[ix];
        sxq[rr][col] = xq[ix];
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int rr = 0; rr < KR; ++rr) {
      float pa[BS], qa[BS], xa[BS], ya[BS];
#pragma unroll
      for (int a = 0; a < BS; ++a) {
        pa[a] = sp[rr][ib + 16 * a];
        qa[a] = sq[rr][ib + 16 * a];
        xa[a] = sxp[rr][jb + 16 * a];
        ya[a] = sxq[rr][jb + 16 * a];
      }
#pragma unroll
      for (int a = 0; a < BS; ++a)
#pragma unroll
        for (int b = 0; b < BS; ++b) acc[a][b] = fmaf(pa[a], xa[b], fmaf(qa[a], ya[b], acc[a][b]));
    }
  }
  const float* af = alpha + ((long long)bh * F + f) * D;
#pragma unroll
  for (int a = 0; a < BS; ++a) {
    const float ra = SANA ? -cc * af[ib + 16 * a] : -cc;
#pragma unroll
    for (int b = 0; b < BS; ++b) dA[fo + (long long)(ib + 16 * a) * D + jb + 16 * b] = ra * acc[a][b];
  }
}

// ---------------------------------------------------------------- statistics
// One workgroup per (frame, b*h): dA + dA^T and dB in LDS; tokens 16 at a
// time, 16 lanes per token (channels l, l + 16, ...). Writes the gradients
// before the convs (fp32) and dbeta.
template <typename T, int D>
__global__ __launch_bounds__(256) void lin_stats_bwd_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ beta,
    const float* __restrict__ conv_k, const float* __restrict__ conv_v,
    const float* __restrict__ dA, const float* __restrict__ dB, float* __restrict__ dkc,
    float* __restrict__ dvc, float* __restrict__ dbeta, int F, int S, int H, long long N) {
  constexpr int LD = D + 1;
  constexpr int TPT = 256 / SB_TT;
  constexpr int CPT = D / TPT;
  __shared__ float g_lds[D * LD];
  __shared__ float b_lds[D * LD];
  __shared__ float kh_lds[SB_TT][D + 4];
  __shared__ float vh_lds[SB_TT][D + 4];
  const int tid = threadIdx.x;
  const int f = blockIdx.x, bh = blockIdx.y;
  const int h = bh % H;
  const long long fo = ((long long)bh * F + f) * D * D;
  for (int x = tid; x < D * D; x += 256) {
    const int i = x / D, j = x % D;
    g_lds[i * LD + j] = dA[fo + x] + dA[fo + (long long)j * D + i];
    b_lds[i * LD + j] = dB[fo + x];
  }
  const int tt = tid / TPT, ln = tid % TPT;
  float wk[CPT][4], wv[CPT][4];
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wk[c][j] = conv_k[((long long)h * D + ln + TPT * c) * 4 + j];
      wv[c][j] = conv_v[((long long)h * D + ln + TPT * c) * 4 + j];
    }
  const long long base = (long long)bh * N * D;
  __syncthreads();
  for (int s0 = 0; s0 < S; s0 += SB_TT) {
    const int s = s0 + tt;
    const bool valid = s < S;
    const long long n = (long long)f * S + s;
    float kc[CPT], kh[CPT], vh[CPT];
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      float ak = 0.0f, av = 0.0f;
      if (valid) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (s - j >= 0) {
            const long long ix = base + (n - j) * D + ln + TPT * c;
            ak = fmaf(wk[c][j], ld_io<T>(k, ix), ak);
            av = fmaf(wv[c][j], ld_io<T>(v, ix), av);
          }
      }
      kc[c] = ak;
      kh[c] = silu_f(ak);
      vh[c] = av;
      ss = fmaf(kh[c], kh[c], ss);
    }
    ss = group_sum<TPT>(ss);
    const float inv = inv_l2(ss);
    const bool clamped = ss <= 1e-24f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      kh[c] *= inv;
      kh_lds[tt][ln + TPT * c] = kh[c];
      vh_lds[tt][ln + TPT * c] = vh[c];
    }
    __syncthreads();
    float gk[CPT], bk[CPT], bv[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) gk[c] = bk[c] = bv[c] = 0.0f;
    for (int m = 0; m < D; ++m) {
      const float km = kh_lds[tt][m], vm = vh_lds[tt][m];
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int i = ln + TPT * c;
        gk[c] = fmaf(g_lds[i * LD + m], km, gk[c]);
        bk[c] = fmaf(b_lds[i * LD + m], km, bk[c]);
        bv[c] = fmaf(b_lds[m * LD + i], vm, bv[c]);
      }
    }
    const float bt = valid ? beta[(long long)bh * N + n] : 0.0f;
    float db = 0.0f, dot = 0.0f;
    float dkh[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      db = fmaf(kh[c], 0.5f * gk[c], db);
      db = fmaf(vh[c], bk[c], db);
      dkh[c] = bt * (gk[c] + bv[c]);
      dot = fmaf(kh[c], dkh[c], dot);
    }
    db = group_sum<TPT>(db);
    dot = group_sum<TPT>(dot);
    if (valid) {
      if (ln == 0) dbeta[(long long)bh * N + n] = db;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const long long ix = base + n * D + ln + TPT * c;
        dkc[ix] = l2_grad(dkh[c], kh[c], inv, dot, clamped) * silu_grad(kc[c]);
        dvc[ix] = bt * bk[c];
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- convs
// One workgroup per (frame, b*h): dk_s = sum_j w_j dkc_{s+j} inside the frame,
// and the frame's part of the tap gradients sum_s dkc_s k_{s-j} (likewise v).
// A thread owns one channel of a contiguous token range and slides two
// four-entry windows along it (dkc_{s..s+3}, k_{s-3..s}): two loads per tensor
// and token.
constexpr int CV_NT = 512;

template <typename T, int D>
__global__ __launch_bounds__(CV_NT) void lin_conv_bwd_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ conv_k,
    const float* __restrict__ conv_v, const float* __restrict__ dkc,
    const float* __restrict__ dvc, T* __restrict__ dk, T* __restrict__ dv,
    float* __restrict__ cpart, int F, int S, int H, long long N, int accum) {
  constexpr int G = CV_NT / D;
  __shared__ float red[G][D][8];
  const int tid = threadIdx.x;
  const int f = blockIdx.x, bh = blockIdx.y;
  const int h = bh % H;
  const int c = tid % D, g0 = tid / D;
  float wk[4], wv[4], pk[4], pv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    wk[j] = conv_k[((long long)h * D + c) * 4 + j];
    wv[j] = conv_v[((long long)h * D + c) * 4 + j];
    pk[j] = pv[j] = 0.0f;
  }
  const int len = (S + G - 1) / G;
  const int sb = min(S, g0 * len), se = min(S, sb + len);
  const long long base = (long long)bh * N * D + (long long)f * S * D + c;
  float gk[4], gv[4], xk[4], xv[4];  // gk[j] = dkc_{s+j}; xk[j] = k_{s-j}
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool fwd = sb + j < S, back = j > 0 && sb - j >= 0;
    gk[j] = fwd ? dkc[base + (long long)(sb + j) * D] : 0.0f;
    gv[j] = fwd ? dvc[base + (long long)(sb + j) * D] : 0.0f;
    xk[j] = back ? ld_io<T>(k, base + (long long)(sb - j) * D) : 0.0f;
    xv[j] = back ? ld_io<T>(v, base + (long long)(sb - j) * D) : 0.0f;
  }
  for (int s = sb; s < se; ++s) {
    const long long ix = base + (long long)s * D;
    xk[0] = ld_io<T>(k, ix);
    xv[0] = ld_io<T>(v, ix);
    float ak = 0.0f, av = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ak = fmaf(wk[j], gk[j], ak);
      av = fmaf(wv[j], gv[j], av);
      pk[j] = fmaf(gk[0], xk[j], pk[j]);
      pv[j] = fmaf(gv[0], xv[j], pv[j]);
    }
    if (accum) {
      ak += ld_io<T>(dk, ix);
      av += ld_io<T>(dv, ix);
    }
    st_io<T>(dk, ix, ak);
    st_io<T>(dv, ix, av);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      gk[j] = gk[j + 1];
      gv[j] = gv[j + 1];
    }
    gk[3] = s + 4 < S ? dkc[ix + 4LL * D] : 0.0f;
    gv[3] = s + 4 < S ? dvc[ix + 4LL * D] : 0.0f;
#pragma unroll
    for (int j = 3; j > 0; --j) {
      xk[j] = xk[j - 1];
      xv[j] = xv[j - 1];
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    red[g0][c][j] = pk[j];
    red[g0][c][4 + j] = pv[j];
  }
  __syncthreads();
  for (int x = tid; x < D * 8; x += CV_NT) {
    float sum = 0.0f;
#pragma unroll
    for (int g = 0; g < G; ++g) sum += red[g][x / 8][x % 8];
    cpart[((long long)bh * F + f) * D * 8 + x] = sum;
  }
}

// Sum of the RMSNorm weight's per-frame partials over every (b, h, frame):
// one workgroup per channel block, a fixed-order tree per channel.
__global__ __launch_bounds__(256) void lin_rms_grad_kernel(const float* __restrict__ dwpart,
                                                           float* __restrict__ drms, int D,
                                                           long long rows) {
  __shared__ float red[256];
  const int j = blockIdx.x;
  float sum = 0.0f;
  for (long long r = threadIdx.x; r < rows; r += 256) sum += dwpart[r * D + j];
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) drms[j] = red[0];
}

// ---------------------------------------------------------------- MFMA variants
// The per-token products of the readout and of the statistics are dense
// contractions of a 16-token tile with the frame's d x d matrices, so for
// d = 64 and 128 they run on fp32 MFMA (v_mfma_f32_16x16x4_f32: fp32 operands
// and accumulation, the VALU kernels' precision). Operand layout of one MFMA:
// A[i][k] from lane i + 16 k, B[k][j] from lane j + 16 k; lane j + 16 g holds
// D[4 g + r][j] in register r. Wave w owns output channels 32 w .. 32 w + 31
// (two 16-column blocks); per-token sums over the channels combine the 16
// lanes of a row group and then the waves through LDS.
namespace {

__device__ __forceinline__ f32x4_t mfma16(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr int MT = 16;  // tokens per MFMA tile

// sum over the 16 lanes of a row group
__device__ __forceinline__ float row_sum16(float x) { return group_sum<16>(x); }

// Eight consecutive channels of one token row: one 16-byte load for bf16
// (rows and the channel offset are 16-byte aligned), eight loads for fp32.
template <typename T>
struct Row8;
template <>
struct Row8<bf16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *(const uint4*)p; }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <>
struct Row8<float> {
  float x[8];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = p[i];
  }
  __device__ __forceinline__ float get(int i) const { return x[i]; }
};

}  // namespace

// Statistics backward on MFMA: gk = (dA + dA^T) k^, bk = dB k^, bv = dB^T v^
// for the 16 tokens of a tile; features staged in LDS by the first half of
// the threads. d / 16 waves (two per SIMD), wave w owning the 16 output
// channels 16 w .. 16 w + 15 of all three products.
template <typename T, int D>
__global__ __launch_bounds__(4 * D) void lin_stats_bwd_mfma_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ beta,
    const float* __restrict__ conv_k, const float* __restrict__ conv_v,
    const float* __restrict__ dA, const float* __restrict__ dB, float* __restrict__ dkc,
    float* __restrict__ dvc, float* __restrict__ dbeta, int F, int S, int H, long long N) {
  constexpr int NT = 4 * D;
  constexpr int NW = D / 16;  // waves, one 16-channel block each
  constexpr int LD = D + 1;
  constexpr int LT = D + 4;
  constexpr int NF = NT / 2;    // feature threads
  constexpr int TPT = NF / MT;  // threads per token: 8 consecutive channels each
  static_assert(TPT * 8 == D, "feature mapping");
  __shared__ float g_lds[D * LD];
  __shared__ float b_lds[D * LD];
  __shared__ __attribute__((aligned(16))) float kh_lds[MT * LT];
  __shared__ __attribute__((aligned(16))) float vh_lds[MT * LT];
  __shared__ __attribute__((aligned(16))) float sg_lds[MT * LT];
  __shared__ float red[NW][MT][2];
  __shared__ float tok_inv[MT];
  __shared__ float tok_beta[MT];
  __shared__ int tok_clamped[MT];
  const int tid = threadIdx.x;
  const int f = blockIdx.x, bh = blockIdx.y;
  const int h = bh % H;
  const long long fo = ((long long)bh * F + f) * D * D;
  for (int x = tid; x < D * D; x += NT) {
    const int i = x / D, j = x % D;
    g_lds[i * LD + j] = dA[fo + x] + dA[fo + (long long)j * D + i];
    b_lds[i * LD + j] = dB[fo + x];
  }
  const bool feat = tid < NF;
  const int tt = (tid % NF) / TPT, ln = tid % TPT;
  const int ch0 = 8 * ln;
  float wk[8][4], wv[8][4];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wk[c][j] = conv_k[((long long)h * D + ch0 + c) * 4 + j];
      wv[c][j] = conv_v[((long long)h * D + ch0 + c) * 4 + j];
    }
  const int lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const long long base = (long long)bh * N * D;
  // raw k, v rows of the conv taps of this thread's token, fetched a tile
  // ahead so their latency overlaps the previous tile's MFMAs
  Row8<T> rk[4], rv[4];
  auto fetch = [&](int s0_) {
    const int s = s0_ + tt;
    if (!feat || s >= S) return;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (s - j >= 0) {
        const long long ix = base + ((long long)f * S + s - j) * D + ch0;
        rk[j].load(k + ix);
        rv[j].load(v + ix);
      }
  };
  fetch(0);
  __syncthreads();
  for (int s0 = 0; s0 < S; s0 += MT) {
    if (feat) {  // features of the tile
      const int s = s0 + tt;
      const bool valid = s < S;
      float kc[8], kh[8], vh[8];
      float ss = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float ak = 0.0f, av = 0.0f;
        if (valid) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (s - j >= 0) {
              ak = fmaf(wk[c][j], rk[j].get(c), ak);
              av = fmaf(wv[c][j], rv[j].get(c), av);
            }
        }
        kc[c] = ak;
        kh[c] = silu_f(ak);
        vh[c] = av;
        ss = fmaf(kh[c], kh[c], ss);
      }
      ss = group_sum<TPT>(ss);
      const float inv = inv_l2(ss);
      const int o = tt * LT + ch0;
      *(float4*)&kh_lds[o] = make_float4(kh[0] * inv, kh[1] * inv, kh[2] * inv, kh[3] * inv);
      *(float4*)&kh_lds[o + 4] = make_float4(kh[4] * inv, kh[5] * inv, kh[6] * inv, kh[7] * inv);
      *(float4*)&vh_lds[o] = make_float4(vh[0], vh[1], vh[2], vh[3]);
      *(float4*)&vh_lds[o + 4] = make_float4(vh[4], vh[5], vh[6], vh[7]);
      *(float4*)&sg_lds[o] = make_float4(silu_grad(kc[0]), silu_grad(kc[1]), silu_grad(kc[2]),
                                         silu_grad(kc[3]));
      *(float4*)&sg_lds[o + 4] = make_float4(silu_grad(kc[4]), silu_grad(kc[5]),
                                             silu_grad(kc[6]), silu_grad(kc[7]));
      if (ln == 0) {
        tok_inv[tt] = inv;
        tok_clamped[tt] = ss <= 1e-24f;
        tok_beta[tt] = valid ? beta[(long long)bh * N + (long long)f * S + s] : 0.0f;
      }
    }
    __syncthreads();
    if (s0 + MT < S) fetch(s0 + MT);
    constexpr int NBW = 1;  // 16-channel blocks per wave
    f32x4_t gk[NBW], bk[NBW], bv[NBW];
#pragma unroll
    for (int b = 0; b < NBW; ++b) gk[b] = bk[b] = bv[b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll  // fully: 9 % faster than by 8
    for (int m0 = 0; m0 < D; m0 += 4) {
      const int m = m0 + lq;
      const float ak = kh_lds[lr * LT + m];
      const float av = vh_lds[lr * LT + m];
#pragma unroll
      for (int b = 0; b < NBW; ++b) {
        const int j = 16 * w + lr;
        gk[b] = mfma16(ak, g_lds[m * LD + j], gk[b]);  // (dA + dA^T) symmetric
        bk[b] = mfma16(ak, b_lds[j * LD + m], bk[b]);  // dB[j][m]
        bv[b] = mfma16(av, b_lds[m * LD + j], bv[b]);  // dB[m][j]
      }
    }
    float db[4], dot[4], dkh[NBW][4], bt[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tk = 4 * lq + r;
      bt[r] = tok_beta[tk];
      db[r] = dot[r] = 0.0f;
#pragma unroll
      for (int b = 0; b < NBW; ++b) {
        const int o = tk * LT + 16 * w + lr;
        const float khv = kh_lds[o], vhv = vh_lds[o];
        db[r] = fmaf(khv, 0.5f * gk[b][r], db[r]);
        db[r] = fmaf(vhv, bk[b][r], db[r]);
        dkh[b][r] = bt[r] * (gk[b][r] + bv[b][r]);
        dot[r] = fmaf(khv, dkh[b][r], dot[r]);
      }
      db[r] = row_sum16(db[r]);
      dot[r] = row_sum16(dot[r]);
      if (lr == 0) {
        red[w][tk][0] = db[r];
        red[w][tk][1] = dot[r];
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tk = 4 * lq + r;
      const int s = s0 + tk;
      if (s >= S) continue;
      float dbt = 0.0f, dt = 0.0f;
#pragma unroll
      for (int x = 0; x < NW; ++x) {
        dbt += red[x][tk][0];
        dt += red[x][tk][1];
      }
      const long long n = (long long)f * S + s;
      if (w == 0 && lr == 0) dbeta[(long long)bh * N + n] = dbt;
      const float inv = tok_inv[tk];
      const bool clamped = tok_clamped[tk] != 0;
#pragma unroll
      for (int b = 0; b < NBW; ++b) {
        const int ch = 16 * w + lr;
        const int o = tk * LT + ch;
        const long long ix = base + n * D + ch;
        dkc[ix] = l2_grad(dkh[b][r], kh_lds[o], inv, dt, clamped) * sg_lds[o];
        dvc[ix] = bt[r] * bk[b][r];
      }
    }
    __syncthreads();
  }
}

// Readout backward on MFMA, per 16-token tile: o = S_t q^ (A: q^ tile, B:
// S_t^T), do from the RMSNorm and gate, dq^ = S_t^T do (A: do tile, B: S_t),
// dS_t += do^T q^ (A: do^T, B: q^; wave w owns rows 32 w .. 32 w + 31 of
// dS_t, all columns, in registers for the whole frame). Two wave groups share
// S_t and take a 16-token tile each per step, so every SIMD holds two waves;
// their dS_t partials are added at the end.
template <typename T, int D>
__global__ __launch_bounds__(4 * D) void lin_readout_bwd_mfma_kernel(
    const T* __restrict__ q, const T* __restrict__ gate, const T* __restrict__ gout,
    const float* __restrict__ alpha, const float* __restrict__ Pst,
    const float* __restrict__ Qst, const float* __restrict__ rms_w, float eps,
    T* __restrict__ dq, T* __restrict__ dgate, float* __restrict__ dSt,
    float* __restrict__ dwpart, int F, int S, int chunk, int radius, long long N, int accum) {
  constexpr int GR = 2;  // wave groups, one token tile each
  constexpr int NT = 2 * D * GR;
  constexpr int NW = D / 32;  // waves per group
  constexpr int NB = D / 16;  // 16-column blocks of dS_t
  constexpr int LD = D + 1;
  constexpr int LT = D + 4;  // (measured: 8 % faster than D + 16)
  constexpr int TPT = NT / (MT * GR);  // threads per token: 8 consecutive channels each
  static_assert(TPT * 8 == D, "feature mapping");
  __shared__ float st_lds[D * LD];
  __shared__ __attribute__((aligned(16))) float qh_lds[GR * MT * LT];
  __shared__ float do_lds[GR * MT * LT];
  __shared__ __attribute__((aligned(16))) float sg_lds[GR * MT * LT];
  __shared__ float red[GR][3][NW][MT];
  __shared__ float tok_inv[GR * MT];
  __shared__ int tok_clamped[GR * MT];
  __shared__ float dec[2][D];
  __shared__ float dwx[D];

  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const int bh = blockIdx.y;
  int lo, hi;
  window_of(t, F, chunk, radius, lo, hi);
  for (int j = tid; j < D; j += NT) {
    const float* al = alpha + (long long)bh * F * D + j;
    float a = 1.0f, b = 1.0f;
    for (int x = lo; x <= t; ++x) a *= al[(long long)x * D];
    for (int x = t; x <= hi; ++x) b *= al[(long long)x * D];
    dec[0][j] = a;
    dec[1][j] = b;
  }
  __syncthreads();
  const float* Pm = Pst + ((long long)bh * (F + 1) + lo) * D * D;      // P_{lo-1}
  const float* Qm = Qst + ((long long)bh * (F + 1) + hi + 1) * D * D;  // Q_{hi+1}
  for (int x = tid; x < D * D; x += NT) {
    const int i = x / D, j = x % D;
    st_lds[i * LD + j] = fmaf(Pm[x], dec[0][j], Qm[x] * dec[1][j]);
  }
  const int tt = tid / TPT, ln = tid % TPT;
  const int lane = tid & 63;
  const int grp = (tid >> 6) / NW, w = (tid >> 6) % NW;  // group, wave within it
  const int lr = lane & 15, lq = lane >> 4;
  float* const qh = qh_lds + grp * MT * LT;
  float* const dob = do_lds + grp * MT * LT;
  float* const sgb = sg_lds + grp * MT * LT;
  float wr[2], dw[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    wr[b] = rms_w ? rms_w[32 * w + 16 * b + lr] : 1.0f;
    dw[b] = 0.0f;
  }
  f32x4_t acc[2][NB];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < NB; ++bj) acc[bi][bj] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const long long base = (long long)bh * N * D;
  const int ch0 = 8 * ln;
  // this thread's 8 channels of its token's q row, fetched a tile ahead
  Row8<T> rq;
  auto fetch = [&](int s0_) {
    const int s = s0_ + tt;
    if (s < S) rq.load(q + base + ((long long)t * S + s) * D + ch0);
  };
  fetch(0);
  __syncthreads();

  for (int s0 = 0; s0 < S; s0 += MT * GR) {
    const int sg0 = s0 + MT * grp;  // this group's tile
    {  // features of both tiles
      const int s = s0 + tt;
      const bool valid = s < S;
      float qv[8], u[8];
      float ss = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        qv[c] = valid ? rq.get(c) : 0.0f;
        u[c] = silu_f(qv[c]);
        ss = fmaf(u[c], u[c], ss);
      }
      ss = group_sum<TPT>(ss);
      const float inv = inv_l2(ss);
      const int o = tt * LT + ch0;
      *(float4*)&qh_lds[o] = make_float4(u[0] * inv, u[1] * inv, u[2] * inv, u[3] * inv);
      *(float4*)&qh_lds[o + 4] = make_float4(u[4] * inv, u[5] * inv, u[6] * inv, u[7] * inv);
      *(float4*)&sg_lds[o] = make_float4(silu_grad(qv[0]), silu_grad(qv[1]), silu_grad(qv[2]),
                                         silu_grad(qv[3]));
      *(float4*)&sg_lds[o + 4] = make_float4(silu_grad(qv[4]), silu_grad(qv[5]),
                                             silu_grad(qv[6]), silu_grad(qv[7]));
      if (ln == 0) {
        tok_inv[tt] = inv;
        tok_clamped[tt] = ss <= 1e-24f;
      }
    }
    __syncthreads();
    // the gate and upstream gradient of this lane's output elements, issued
    // before the next tile's q so the first product hides their latency
    float gtv[2][4], gov[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = sg0 + 4 * lq + r;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const long long ix = base + ((long long)t * S + s) * D + 32 * w + 16 * b + lr;
        gtv[b][r] = s < S ? ld_io<T>(gate, ix) : 0.0f;
        gov[b][r] = s < S ? ld_io<T>(gout, ix) : 0.0f;
      }
    }
    if (s0 + MT * GR < S) fetch(s0 + MT * GR);
    // o = S_t q^
    f32x4_t o[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) o[b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int m0 = 0; m0 < D; m0 += 4) {
      const int m = m0 + lq;
      const float a = qh[lr * LT + m];
#pragma unroll
      for (int b = 0; b < 2; ++b) o[b] = mfma16(a, st_lds[(32 * w + 16 * b + lr) * LD + m], o[b]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float ms = 0.0f;
#pragma unroll
      for (int b = 0; b < 2; ++b) ms = fmaf(o[b][r], o[b][r], ms);
      ms = row_sum16(ms);
      if (lr == 0) red[grp][0][w][4 * lq + r] = ms;
    }
    __syncthreads();
    float rinv[4], z[2][4], dz[2][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tk = 4 * lq + r;
      const int s = sg0 + tk;
      const bool valid = s < S;
      float ms = 0.0f;
#pragma unroll
      for (int x = 0; x < NW; ++x) ms += red[grp][0][x][tk];
      rinv[r] = 1.0f / sqrtf(ms / D + eps);
      float dzz = 0.0f;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const long long ix = base + ((long long)t * S + s) * D + 32 * w + 16 * b + lr;
        const float go = gov[b][r];
        const float sg = sigmoid_f(gtv[b][r]);
        z[b][r] = o[b][r] * rinv[r];
        if (valid) st_io<T>(dgate, ix, go * z[b][r] * wr[b] * sg * (1.0f - sg));
        dw[b] = fmaf(go * sg, z[b][r], dw[b]);
        dz[b][r] = go * wr[b] * sg;
        dzz = fmaf(dz[b][r], z[b][r], dzz);
      }
      dzz = row_sum16(dzz);
      if (lr == 0) red[grp][1][w][tk] = dzz;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tk = 4 * lq + r;
      float mz = 0.0f;
#pragma unroll
      for (int x = 0; x < NW; ++x) mz += red[grp][1][x][tk];
      mz /= D;
#pragma unroll
      for (int b = 0; b < 2; ++b)
        dob[tk * LT + 32 * w + 16 * b + lr] = rinv[r] * (dz[b][r] - z[b][r] * mz);
    }
    __syncthreads();
    // dq^ = S_t^T do
    f32x4_t g[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) g[b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int i0 = 0; i0 < D; i0 += 4) {
      const int i = i0 + lq;
      const float a = dob[lr * LT + i];
#pragma unroll
      for (int b = 0; b < 2; ++b) g[b] = mfma16(a, st_lds[i * LD + 32 * w + 16 * b + lr], g[b]);
    }
    // dS_t += do^T q^ over the tile's tokens
#pragma unroll
    for (int k0 = 0; k0 < MT; k0 += 4) {
      const int tk = k0 + lq;
      float a[2], bq[NB];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) a[bi] = dob[tk * LT + 32 * w + 16 * bi + lr];
#pragma unroll
      for (int bj = 0; bj < NB; ++bj) bq[bj] = qh[tk * LT + 16 * bj + lr];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < NB; ++bj) acc[bi][bj] = mfma16(a[bi], bq[bj], acc[bi][bj]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tk = 4 * lq + r;
      float dt = 0.0f;
#pragma unroll
      for (int b = 0; b < 2; ++b) dt = fmaf(qh[tk * LT + 32 * w + 16 * b + lr], g[b][r], dt);
      dt = row_sum16(dt);
      if (lr == 0) red[grp][2][w][tk] = dt;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tk = 4 * lq + r;
      const int s = sg0 + tk;
      if (s >= S) continue;
      float dt = 0.0f;
#pragma unroll
      for (int x = 0; x < NW; ++x) dt += red[grp][2][x][tk];
      const float inv = tok_inv[grp * MT + tk];
      const bool clamped = tok_clamped[grp * MT + tk] != 0;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int ch = 32 * w + 16 * b + lr;
        const int o2 = tk * LT + ch;
        const long long ix = base + ((long long)t * S + s) * D + ch;
        st_io<T>(dq, ix,
                 l2_grad(g[b][r], qh[o2], inv, dt, clamped) * sgb[o2] +
                     (accum ? ld_io<T>(dq, ix) : 0.0f));
      }
    }
    __syncthreads();
  }
  // group 1 hands its dS_t and dw partials to group 0 through LDS (S_t is no
  // longer read after the loop's last barrier)
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    dw[b] += __shfl_xor(dw[b], 16);
    dw[b] += __shfl_xor(dw[b], 32);
  }
  if (grp == 1) {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < NB; ++bj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          st_lds[(32 * w + 16 * bi + 4 * lq + r) * D + 16 * bj + lr] = acc[bi][bj][r];
    if (lq == 0) {
#pragma unroll
      for (int b = 0; b < 2; ++b) dwx[32 * w + 16 * b + lr] = dw[b];
    }
  }
  __syncthreads();
  if (grp == 0) {
    float* ds = dSt + ((long long)bh * F + t) * D * D;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int bj = 0; bj < NB; ++bj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int o = (32 * w + 16 * bi + 4 * lq + r) * D + 16 * bj + lr;
          ds[o] = acc[bi][bj][r] + st_lds[o];
        }
    if (lq == 0) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int ch = 32 * w + 16 * b + lr;
        dwpart[((long long)bh * F + t) * D + ch] = dw[b] + dwx[ch];
      }
    }
  }
}

// ---------------------------------------------------------------- dalpha
// dalpha_f = the scans' part + the gather's: a_t and b_t are products over
// frames of the window, so frame f's factor gets da_t (db_t) times the
// product of the other factors.
template <int D>
__global__ __launch_bounds__(256) void lin_alpha_grad_kernel(
    const float* __restrict__ alpha, const float* __restrict__ gab,
    const float* __restrict__ dal, float* __restrict__ dalpha, int F, int chunk, int radius,
    int BH) {
  const long long idx = blockIdx.x * 256LL + threadIdx.x;
  if (idx >= (long long)BH * F * D) return;
  const int j = (int)(idx % D);
  const long long rf = idx / D;
  const int f = (int)(rf % F);
  const long long bh = rf / F;
  const float* al = alpha + bh * F * D + j;
  const float* ga = gab + bh * F * D + j;
  const float* gb = gab + ((long long)BH + bh) * F * D + j;
  float acc = dal[idx];
  const long long W = min((long long)F, (2LL * radius + 2) * chunk);
  const int t0 = (int)max(0LL, f - W), t1 = (int)min((long long)F - 1, f + W);
  for (int t = t0; t <= t1; ++t) {
    int lo, hi;
    window_of(t, F, chunk, radius, lo, hi);
    if (lo <= f && f <= t) {
      float pr = 1.0f;
      for (int x = lo; x <= t; ++x)
        if (x != f) pr *= al[(long long)x * D];
      acc = fmaf(ga[(long long)t * D], pr, acc);
    }
    if (t <= f && f <= hi) {
      float pr = 1.0f;
      for (int x = t; x <= hi; ++x)
        if (x != f) pr *= al[(long long)x * D];
      acc = fmaf(gb[(long long)t * D], pr, acc);
    }
  }
  dalpha[idx] = acc;
}

// ---------------------------------------------------------------- parameters
// Per-head conv taps (sum over batch and frames) and dS_text = text_scale
// (lam_P + lam_Q); one thread per output.
__global__ __launch_bounds__(256) void lin_param_grad_kernel(
    const float* __restrict__ cpart, const float* __restrict__ lam0, float* __restrict__ dconv_k,
    float* __restrict__ dconv_v, float* __restrict__ dtext, float text_scale, int B, int H, int D,
    int F) {
  const long long idx = blockIdx.x * 256LL + threadIdx.x;
  const long long BH = (long long)B * H;
  const long long n_conv = (long long)H * D * 8;
  const long long n_text = BH * D * D;
  if (idx < n_conv) {
    const int h = (int)(idx / (D * 8));
    const int x = (int)(idx % (D * 8));  // channel * 8 + tap (k: 0..3, v: 4..7)
    float sum = 0.0f;
    for (int b = 0; b < B; ++b)
      for (int f = 0; f < F; ++f)
        sum += cpart[(((long long)b * H + h) * F + f) * D * 8 + x];
    const int ch = x / 8, tap = x % 8;
    float* dst = tap < 4 ? dconv_k : dconv_v;
    dst[((long long)h * D + ch) * 4 + (tap & 3)] = sum;
  } else if (idx < n_conv + n_text) {
    const long long x = idx - n_conv;
    if (dtext) dtext[x] = text_scale * (lam0[x] + lam0[n_text + x]);
  }
}

// ---------------------------------------------------------------- launch sequence
#define LB_SWITCH_D(MACRO)          \
  switch (g.d) {                    \
    case 16: MACRO(16); break;      \
    case 32: MACRO(32); break;      \
    case 64: MACRO(64); break;      \
    default: MACRO(128); break;     \
  }

hipError_t launch_linear_bwd(const Geom& g, int dtype, int stage, const LinBwdArgs& a,
                             hipStream_t st) {
  const int BH = g.B * g.H;
  const bool sana = a.rule == HWA_RULE_SANA_SCALED;
  const float cc = a.rule == HWA_RULE_VDN_SOLVE ? 1.0f : a.c * a.c;
  // dB_f's factor: c1 of X_f = S D + c1 B_f (vdn rules), c2 of + c2 B_f (SANA)
  const float cb = a.rule == HWA_RULE_VDN_SOLVE ? 1.0f : a.c;
  const bool bf = dtype == HWA_BF16;
  hipError_t e = hipSuccess;
  switch (stage) {
    case 0: {  // recompute: statistics, inverses, every frame's states
      e = launch_stats(g, dtype, a.k, a.v, a.beta, a.conv_k, a.conv_v, true, a.A, a.Bm, st);
      if (e != hipSuccess) return e;
      e = launch_update_f32(g, !sana, cc, a.A, a.M, st);
      if (e != hipSuccess) return e;
      Geom g1 = g;
      g1.chunk = 1;
      g1.nch = g.F;
      // the forward's own scan for the call's dtype (bf16: split-bf16 MFMA,
      // about 16 significant bits per product; fp32: fp32)
      e = launch_scan(g1, dtype, a.rule, a.c, a.A, a.Bm, a.M, a.alpha, a.text_state,
                      a.text_scale, a.Pst, a.Qst, a.E, st);
      if (e != hipSuccess) return e;
      const long long rows = (long long)BH * (g.F + 1) * g.d;
      const long long work = 2 * rows * g.d;
      const unsigned blocks = (unsigned)min(8192LL, (work + 255) / 256);
      hipLaunchKernelGGL(fold_exp_kernel, dim3(blocks), dim3(256), 0, st, a.Pst, a.Qst, a.E,
                         rows, g.d);
      break;
    }
    case 1: {  // readout
      dim3 grid(g.F, BH);
#define RB(DD)                                                                           \
  if (bf)                                                                                \
    hipLaunchKernelGGL((lin_readout_bwd_kernel<bf16_t, DD>), grid, dim3(256), 0, st,      \
                       (const bf16_t*)a.q, (const bf16_t*)a.gate, (const bf16_t*)a.d_o,   \
                       a.alpha, a.Pst, a.Qst, a.rms_w, a.eps, (bf16_t*)a.dq,              \
                       (bf16_t*)a.dgate, a.dSt, a.dwpart, g.F, g.S, g.chunk, g.radius, g.N, a.acc); \
  else                                                                                   \
    hipLaunchKernelGGL((lin_readout_bwd_kernel<float, DD>), grid, dim3(256), 0, st,       \
                       (const float*)a.q, (const float*)a.gate, (const float*)a.d_o,      \
                       a.alpha, a.Pst, a.Qst, a.rms_w, a.eps, (float*)a.dq,               \
                       (float*)a.dgate, a.dSt, a.dwpart, g.F, g.S, g.chunk, g.radius, g.N, a.acc);
#define RBM(DD)                                                                          \
  if (bf)                                                                                \
    hipLaunchKernelGGL((lin_readout_bwd_mfma_kernel<bf16_t, DD>), grid, dim3(4 * DD), 0, st, \
                       (const bf16_t*)a.q, (const bf16_t*)a.gate, (const bf16_t*)a.d_o,   \
                       a.alpha, a.Pst, a.Qst, a.rms_w, a.eps, (bf16_t*)a.dq,              \
                       (bf16_t*)a.dgate, a.dSt, a.dwpart, g.F, g.S, g.chunk, g.radius, g.N, a.acc); \
  else                                                                                   \
    hipLaunchKernelGGL((lin_readout_bwd_mfma_kernel<float, DD>), grid, dim3(4 * DD), 0, st, \
                       (const float*)a.q, (const float*)a.gate, (const float*)a.d_o,      \
                       a.alpha, a.Pst, a.Qst, a.rms_w, a.eps, (float*)a.dq,               \
                       (float*)a.dgate, a.dSt, a.dwpart, g.F, g.S, g.chunk, g.radius, g.N, a.acc);
      switch (g.d) {
        case 16: RB(16); break;
        case 32: RB(32); break;
        case 64: RBM(64); break;
        default: RBM(128); break;
      }
#undef RBM
#undef RB
      break;
    }
    case 2: {  // gather, adjoint scans, frame gradients
      {
        dim3 grid(g.nch + 1, 2, BH);
#define GB(DD)                                                                       \
  hipLaunchKernelGGL(lin_gather_bwd_kernel<DD>, grid, dim3(256), 0, st, a.dSt, a.alpha, \
                     a.Pst, a.Qst, a.dbank, a.gab, g.F, g.chunk, g.radius, g.nch, BH);
        LB_SWITCH_D(GB)
#undef GB
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      {
        dim3 grid(g.d / AJ_R, 2, BH);
#define AJ(DD)                                                                          \
  hipLaunchKernelGGL(lin_adjoint_kernel<DD>, grid, dim3(256), 0, st, a.M, a.alpha, a.dbank, \
                     a.dXP, a.dXQ, a.lam0, g.F, g.chunk, g.nch, BH);
        LB_SWITCH_D(AJ)
#undef AJ
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      {
        dim3 grid(g.F, BH);
#define FG(DD)                                                                            \
  if (sana)                                                                                \
    hipLaunchKernelGGL((lin_frame_grad_kernel<DD, true>), grid, dim3(256), 0, st, a.Pst,     \
                       a.Qst, a.dXP, a.dXQ, cc, cb, a.alpha, a.dbank, g.chunk, g.nch, BH,  \
                       a.A, a.Bm, a.dal, g.F);                                              \
  else                                                                                     \
    hipLaunchKernelGGL((lin_frame_grad_kernel<DD, false>), grid, dim3(256), 0, st, a.Pst,    \
                       a.Qst, a.dXP, a.dXQ, cc, cb, a.alpha, a.dbank, g.chunk, g.nch, BH,  \
                       a.A, a.Bm, a.dal, g.F);
        LB_SWITCH_D(FG)
#undef FG
      }
      break;
    }
    case 3: {  // statistics and features
      dim3 grid(g.F, BH);
#define SB(DD)                                                                              \
  if (bf)                                                                                   \
    hipLaunchKernelGGL((lin_stats_bwd_kernel<bf16_t, DD>), grid, dim3(256), 0, st,          \
                       (const bf16_t*)a.k, (const bf16_t*)a.v, a.beta, a.conv_k, a.conv_v,   \
                       a.A, a.Bm, a.dkc, a.dvc, a.dbeta, g.F, g.S, g.H, g.N);               \
  else                                                                                      \
    hipLaunchKernelGGL((lin_stats_bwd_kernel<float, DD>), grid, dim3(256), 0, st,           \
                       (const float*)a.k, (const float*)a.v, a.beta, a.conv_k, a.conv_v,     \
                       a.A, a.Bm, a.dkc, a.dvc, a.dbeta, g.F, g.S, g.H, g.N);
#define SBM(DD)                                                                             \
  if (bf)                                                                                   \
    hipLaunchKernelGGL((lin_stats_bwd_mfma_kernel<bf16_t, DD>), grid, dim3(4 * DD), 0, st,  \
                       (const bf16_t*)a.k, (const bf16_t*)a.v, a.beta, a.conv_k, a.conv_v,   \
                       a.A, a.Bm, a.dkc, a.dvc, a.dbeta, g.F, g.S, g.H, g.N);               \
  else                                                                                      \
    hipLaunchKernelGGL((lin_stats_bwd_mfma_kernel<float, DD>), grid, dim3(4 * DD), 0, st,   \
                       (const float*)a.k, (const float*)a.v, a.beta, a.conv_k, a.conv_v,     \
                       a.A, a.Bm, a.dkc, a.dvc, a.dbeta, g.F, g.S, g.H, g.N);
      switch (g.d) {
        case 16: SB(16); break;
        case 32: SB(32); break;
        case 64: SBM(64); break;
        default: SBM(128); break;
      }
#undef SBM
#undef SB
      break;
    }
    case 4: {  // convs, dalpha, parameter sums
      {
        dim3 grid(g.F, BH);
#define CB(DD)                                                                              \
  if (bf)                                                                                   \
    hipLaunchKernelGGL((lin_conv_bwd_kernel<bf16_t, DD>), grid, dim3(CV_NT), 0, st,           \
                       (const bf16_t*)a.k, (const bf16_t*)a.v, a.conv_k, a.conv_v, a.dkc,    \
                       a.dvc, (bf16_t*)a.dk, (bf16_t*)a.dv, a.cpart, g.F, g.S, g.H, g.N, a.acc);   \
  else                                                                                      \
    hipLaunchKernelGGL((lin_conv_bwd_kernel<float, DD>), grid, dim3(CV_NT), 0, st,            \
                       (const float*)a.k, (const float*)a.v, a.conv_k, a.conv_v, a.dkc,     \
                       a.dvc, (float*)a.dk, (float*)a.dv, a.cpart, g.F, g.S, g.H, g.N, a.acc);
        LB_SWITCH_D(CB)
#undef CB
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      {
        const long long n = (long long)BH * g.F * g.d;
        dim3 grid((unsigned)((n + 255) / 256));
#define AG(DD)                                                                            \
  hipLaunchKernelGGL(lin_alpha_grad_kernel<DD>, grid, dim3(256), 0, st, a.alpha, a.gab,    \
                     a.dal, a.dalpha, g.F, g.chunk, g.radius, BH);
        LB_SWITCH_D(AG)
#undef AG
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      {
        const long long n = (long long)g.H * g.d * 8 + (long long)BH * g.d * g.d;
        hipLaunchKernelGGL(lin_param_grad_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256),
                           0, st, a.cpart, a.lam0, a.dconv_k, a.dconv_v, a.dtext, a.text_scale,
                           g.B, g.H, g.d, g.F);
        if (a.drms) {
          if ((e = hipGetLastError()) != hipSuccess) return e;
          hipLaunchKernelGGL(lin_rms_grad_kernel, dim3(g.d), dim3(256), 0, st, a.dwpart, a.drms,
                             g.d, (long long)BH * g.F);
        }
      }
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

#undef LB_SWITCH_D

}  // namespace hwa
