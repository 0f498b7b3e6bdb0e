// Finishing kernels: deterministic cross-workgroup reductions of the forward sweep's per-split partials into
// the loss, the per-row losses and dH, and the cotangent scaling of dH in the backward.
//
// Per valid row r the forward sweep leaves, for every vocabulary split, (e, p): e = sum over the split's items
// of softplus(z) - ln 2 - z and p = sum of z over the row's positives in the split. With the row's logit sum
// sum_v z_rv = H[r] . (sum_v E[v]) (a rank-1 identity, evaluated in float64), the unnormalised row loss of
// "Cut Binary Cross Entropy" Eq. (2)-(3) is
//   V ln 2 + H[r].sum_v E[v] + sum_splits e - sum_splits p,
// and dH[r] = s * w_r * (sum_splits dH_part + (1/2) sum_v E[v]) (Eq. (4) with sigma split as
// (sigma - 1/2) + 1/2). The loss is s * sum_r w_r * (row loss), rows added in compacted order in float64; w_r
// is the row's weight (1 without weights) and s = 1 / (W V).
// With Cut Metrics (Section III-D) the sweep also leaves, per split, the counts of logits predicted positive
// (z > 0), of positives predicted positive and of positives; TP, FP, FN and TN follow by subtraction.
#include "common.h"

namespace cutbce {

__device__ inline int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

__device__ inline double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ inline int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Positives of compact row k gathered here (when the forward sweep ran without them): the row's ids in
// rptr[k] (clamped range), those in [0, V) and not repeated earlier in the row, give S = sum_{v in P_r} E[v];
// then sum_{v in P_r} z_rv = H[r] . S (float64) and the sparse part of dH is -S. One wave per row: the lanes form
// groups of D * sizeof(T) / 16 lanes, each lane loading 16 bytes of an E row; group g takes the positives
// g, g + NG, ... in row order, and the groups' sums are added in group order (deterministic).
template <typename T>
__device__ inline void gather_positives(const int2* __restrict__ rptr, const int32_t* __restrict__ ids,
                                        const T* __restrict__ E, int64_t V, int D, int64_t k, int lane, float* sh,
                                        float* S /* [D / 64], d = lane + 64 i */) {
  constexpr int EPL = 16 / sizeof(T);  // elements per 16-byte load
  const int lpr = D / EPL;              // lanes per E row (8 ... 64)
  const int ng = 64 / lpr, g = lane / lpr, sub = lane % lpr;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  const int2 rg = rptr[k];
  for (int q0 = rg.x; q0 < rg.y; q0 += 64) {  // uniform
    const int q = q0 + lane;
    const int v = q < rg.y ? ids[q] : -1;
    bool keep = v >= 0 && v < V;
    // (every lane runs every shuffle: a shuffle reads nothing from lanes that skip it)
    for (int q1 = rg.x; q1 < q0; q1 += 64) {  // earlier chunks of the row
      const int u = ids[q1 + lane];           // q1 + 63 < q0 <= rg.y - 1: inside the row
      for (int j = 0; j < 64; ++j) {
        const int uj = __shfl(u, j, 64);
        keep = keep & (uj != v);
      }
    }
    const int nq = rg.y - q0 < 64 ? rg.y - q0 : 64;  // ids in this chunk (uniform)
    for (int j = 0; j + 1 < nq; ++j) {              // earlier lanes of this chunk
      const int u = __shfl(v, j, 64);
      keep = keep & !(j < lane && u == v);
    }
    uint64_t m = __ballot(keep);
    while (m) {  // uniform: kRounds rounds of up to ng positives each (one per group), their loads issued together
      constexpr int kRounds = 8;
      int vv[kRounds];
      bool has[kRounds];
#pragma unroll
      for (int u = 0; u < kRounds; ++u) {
        int src = -1;
        for (int gg = 0; gg < ng && m; ++gg) {
          const int b = __builtin_ctzll(m);
          m &= m - 1;
          if (g == gg) src = b;
        }
        vv[u] = __shfl(v, src < 0 ? 0 : src, 64);
        has[u] = src >= 0;
      }
      u32x4 raw[kRounds];
#pragma unroll
      for (int u = 0; u < kRounds; ++u)
        raw[u] = has[u] ? *(const u32x4*)(E + (int64_t)vv[u] * D + sub * EPL) : u32x4{0u, 0u, 0u, 0u};
      // added round by round: each group takes its positives in row order, as one round at a time would
#pragma unroll
      for (int u = 0; u < kRounds; ++u)
        if (has[u]) {
          const T* x = (const T*)&raw[u];
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] += (float)x[e];
        }
    }
  }
  // the groups' sums, added in group order
#pragma unroll
  for (int e = 0; e < EPL; ++e) sh[g * D + sub * EPL + e] = acc[e];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int i = 0, d = lane; d < D; ++i, d += 64) {
    float t = 0.f;
    for (int gg = 0; gg < ng; ++gg) t += sh[gg * D + d];
    S[i] = t;
  }
}

template <typename T>
__global__ void __launch_bounds__(256) k_rows_finish(const Ctl* __restrict__ ctl, const T* __restrict__ H,
                                                     const uint8_t* __restrict__ mask,
                                                     const int32_t* __restrict__ compact_of,
                                                     const float* __restrict__ wc,
                                                     const float* __restrict__ dhpart,
                                                     const float2* __restrict__ rowpart,
                                                     const int4* __restrict__ metpart,
                                                     const double* __restrict__ sumE, int64_t R, int64_t V, int D,
                                                     int RW, float* __restrict__ row_loss,
                                                     double* __restrict__ rowloss_c, float* __restrict__ dh_out,
                                                     int32_t* __restrict__ metrics, const int2* __restrict__ rptr,
                                                     const int32_t* __restrict__ ids, const T* __restrict__ E,
                                                     const uint8_t* __restrict__ rowform) {
  __shared__ float sh_pos[4][512];  // per wave: the positive groups' partial sums (at most 512 floats)
  const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = lane_id();
  if (r >= R) return;
  if (mask[r] == 0) {
    if (row_loss && lane == 0) row_loss[r] = 0.f;
    if (metrics && lane < 4) metrics[r * 4 + lane] = 0;
    if (dh_out)
      for (int d = lane; d < D; d += 64) dh_out[r * D + d] = 0.f;
    return;
  }
  const int k = compact_of[r];
  const int S = ctl->splits;
  const int Tt = (ctl->n_valid + RW - 1) / RW;
  const int t = k / RW, loc = k % RW;
  const double w = (double)wc[k];
  const double sw = ctl->scale * w;  // s w_r (= s exactly for unit weights)
  float Sp[8];                       // sum of the row's positives' E rows (d = lane + 64 i), gathered here
#pragma unroll
  for (int i = 0; i < 8; ++i) Sp[i] = 0.f;
  if (E) gather_positives<T>(rptr, ids, E, V, D, k, lane, sh_pos[threadIdx.x / 64], Sp);
  if (dh_out) {
    // split s's partial of (row tile t, row loc) sits at ((s Tt + t) RW + loc) D; the splits are added in order,
    // eight loads issued before their adds
    const int64_t stride = (int64_t)Tt * RW * D;
    for (int i = 0, d = lane; d < D; ++i, d += 64) {
      const float* src = dhpart + ((int64_t)t * RW + loc) * D + d;
      double acc = 0.0;
      for (int s0 = 0; s0 < S; s0 += 8) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = src[(int64_t)min(s0 + j, S - 1) * stride];  // past S: unused
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (s0 + j < S) acc += (double)x[j];
      }
      dh_out[r * D + d] = (float)(sw * (acc + 0.5 * sumE[d] - (double)Sp[i]));
    }
  }
  double e = 0.0, p = 0.0;
  for (int s = lane; s < S; s += 64) {
    const float2 q = rowpart[(int64_t)(s * Tt + t) * RW + loc];
    e += q.x;
    p += q.y;
  }
  double zs = 0.0, pg = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // d = lane + 64 i < D <= 512
    const int d = lane + 64 * i;
    if (d < D) {
      const double h = (double)(float)H[r * D + d];
      zs += h * sumE[d];
      pg += h * (double)Sp[i];
    }
  }
  e = wave_sum(e);
  p = wave_sum(p) + wave_sum(pg);
  zs = wave_sum(zs);
  if (metrics) {
    // Cut Metrics: predicted positive (z > 0), true positives, positives, summed over the splits
    int np = 0, tp = 0, npos = 0;
    for (int s = lane; s < S; s += 64) {
      const int4 q = metpart[(int64_t)(s * Tt + t) * RW + loc];
      np += q.x;
      tp += q.y;
      npos += q.z;
    }
    np = wave_sum_i(np);
    tp = wave_sum_i(tp);
    npos = wave_sum_i(npos);
    const int fp = np - tp, fn = npos - tp, tn = (int)(V - tp - fp - fn);
    if (lane < 4) metrics[r * 4 + lane] = lane == 0 ? tp : lane == 1 ? fp : lane == 2 ? fn : tn;
  }
  // rows whose forward waves took the polynomial epilogue summed log cosh(z/2) only: their -z/2 terms, summed over
  // every item and split, are the rank-1 -H[r].sum_v E[v] / 2
  const bool poly = rowform && rowform[k];
  const double rl = (double)V * 0.69314718055994530942 + (poly ? 0.5 * zs : zs) + e - p;
  if (lane == 0) {
    if (row_loss) row_loss[r] = (float)rl;
    rowloss_c[k] = w * rl;
  }
}

__global__ void __launch_bounds__(1024) k_loss_final(const Ctl* __restrict__ ctl, const double* __restrict__ rl,
                                                     float* __restrict__ loss) {
  __shared__ double sh[16];
  const int n = ctl->n_valid;
  double s = 0.0;
  for (int k = threadIdx.x; k < n; k += 1024) s += rl[k];
  s = wave_sum(s);
  if (lane_id() == 0) sh[threadIdx.x / 64] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int w = 0; w < 16; ++w) tot += sh[w];
    loss[0] = (float)(ctl->scale * tot);
  }
}

hipError_t launch_rows_finish(const Layout& L, char* ws, const void* H, const uint8_t* mask, float* loss,
                              float* row_loss, float* dh_out, bool with_dh, int32_t* metrics, const void* E,
                              const int32_t* item_ids, hipStream_t st) {
  const int2* rptr = (const int2*)(ws + L.off_rptr);
  const unsigned blocks = (unsigned)((L.R + 3) / 4);
  const Ctl* ctl = (const Ctl*)(ws + L.off_ctl);
  if (L.dtype == 1) {
    hipLaunchKernelGGL(k_rows_finish<__bf16>, dim3(blocks), dim3(256), 0, st, ctl, (const __bf16*)H, mask,
                       (const int32_t*)(ws + L.off_compact_of), (const float*)(ws + L.off_wc),
                       (const float*)(ws + L.off_dhpart),
                       (const float2*)(ws + L.off_rowpart), (const int4*)(ws + L.off_metpart),
                       (const double*)(ws + L.off_sumE), L.R, L.V, L.D, L.rows_per_wg, row_loss,
                       (double*)(ws + L.off_rowloss), with_dh ? dh_out : nullptr, metrics, rptr, item_ids,
                       (const __bf16*)E, evp_is_f16(L.dtype, L.D) ? (const uint8_t*)(ws + L.off_rowform) : nullptr);
  } else {
    hipLaunchKernelGGL(k_rows_finish<float>, dim3(blocks), dim3(256), 0, st, ctl, (const float*)H, mask,
                       (const int32_t*)(ws + L.off_compact_of), (const float*)(ws + L.off_wc),
                       (const float*)(ws + L.off_dhpart),
                       (const float2*)(ws + L.off_rowpart), (const int4*)(ws + L.off_metpart),
                       (const double*)(ws + L.off_sumE), L.R, L.V, L.D, L.rows_per_wg, row_loss,
                       (double*)(ws + L.off_rowloss), with_dh ? dh_out : nullptr, metrics, rptr, item_ids,
                       (const float*)E, evp_is_f16(L.dtype, L.D) ? (const uint8_t*)(ws + L.off_rowform) : nullptr);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !loss) return e;
  hipLaunchKernelGGL(k_loss_final, dim3(1), dim3(1024), 0, st, ctl, (const double*)(ws + L.off_rowloss), loss);
  return hipGetLastError();
}

// Scoring finish (full-vocabulary top-k, the evaluation of "Cut Binary Cross Entropy" Section III-E): one wave
// per row merges the S per-split top-KT lists of the forward sweep into the row's k best items -- larger
// logit first, smaller item id among equal logits -- by k rounds of a wave-wide selection over candidates held
// in registers, and counts how many of them are positives of the row (Hit@k: the row is a hit when the count is
// non-zero). Masked rows get ids -1, logits -inf and count 0.
constexpr int kMaxCandPerLane = kMaxSplits * kTopKMax / 64;  // S * KT / 64 with S <= 64, KT <= kTopKMax

__device__ inline bool ranks_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ void __launch_bounds__(256) k_topk_finish(const Ctl* __restrict__ ctl, const uint8_t* __restrict__ mask,
                                                     const int32_t* __restrict__ compact_of,
                                                     const int2* __restrict__ rptr,
                                                     const int32_t* __restrict__ item_ids,
                                                     const float* __restrict__ topv, const int32_t* __restrict__ topi,
                                                     int64_t R, int RW, int KT, int k, float* __restrict__ vals,
                                                     int32_t* __restrict__ ids, int32_t* __restrict__ hits) {
  const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = lane_id();
  if (r >= R) return;
  if (mask[r] == 0) {
    if (lane < k) {
      vals[r * k + lane] = -__builtin_inff();
      ids[r * k + lane] = -1;
    }
    if (hits && lane == 0) hits[r] = 0;
    return;
  }
  const int kc = compact_of[r];
  const int S = ctl->splits;
  const int Tt = (ctl->n_valid + RW - 1) / RW;
  const int t = kc / RW, loc = kc % RW;
  const int nc = S * KT;
  float cv[kMaxCandPerLane];
  int ci[kMaxCandPerLane];
#pragma unroll
  for (int m = 0; m < kMaxCandPerLane; ++m) {
    const int c = lane + 64 * m;
    cv[m] = -__builtin_inff();
    ci[m] = -1;
    if (c < nc) {
      const int64_t at = ((int64_t)((c / KT) * Tt + t) * RW + loc) * KT + c % KT;
      cv[m] = topv[at];
      ci[m] = topi[at];
    }
  }
  float last_v = __builtin_inff(), sel_v = -__builtin_inff();
  int last_i = -1, sel_i = -1;
  for (int q = 0; q < k; ++q) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll
    for (int m = 0; m < kMaxCandPerLane; ++m) {
      const bool after = ci[m] >= 0 && ranks_before(last_v, last_i, cv[m], ci[m]);
      if (after && ranks_before(cv[m], ci[m], bv, bi)) {
        bv = cv[m];
        bi = ci[m];
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ranks_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == q) {
      sel_v = bv;
      sel_i = bi;
    }
    last_v = bv;
    last_i = bi;
  }
  if (lane < k) {
    vals[r * k + lane] = sel_v;
    ids[r * k + lane] = sel_i;
  }
  if (hits) {
    bool hit = false;
    if (lane < k) {
      const int2 rp = rptr[kc];
      for (int p = rp.x; p < rp.y; ++p) hit |= item_ids[p] == sel_i;
    }
    const uint64_t b = __ballot(hit);
    if (lane == 0) hits[r] = __popcll(b);
  }
}

hipError_t launch_topk_finish(const Layout& L, char* ws, const uint8_t* mask, const int32_t* item_ids, int kt, int k,
                              float* vals, int32_t* ids, int32_t* hits, hipStream_t st) {
  const unsigned blocks = (unsigned)((L.R + 3) / 4);
  hipLaunchKernelGGL(k_topk_finish, dim3(blocks), dim3(256), 0, st, (const Ctl*)(ws + L.off_ctl), mask,
                     (const int32_t*)(ws + L.off_compact_of), (const int2*)(ws + L.off_rptr), item_ids,
                     (const float*)(ws + L.off_dhpart),
                     (const int32_t*)(ws + L.off_dhpart) + (size_t)L.part_rows * kt, L.R, L.rows_per_wg, kt, k,
                     vals, ids, hits);
  return hipGetLastError();
}

template <typename T>
__global__ void k_scale_dh(const float* __restrict__ src, const float* __restrict__ g, T* __restrict__ dst,
                           int64_t n) {
  const float gg = g[0];
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = (T)(gg * src[i]);
}

hipError_t launch_scale_dh(const Layout& L, const float* src, const float* grad_loss, void* dH, hipStream_t st) {
  const int64_t n = L.R * L.D;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (L.dtype == 1)
    hipLaunchKernelGGL(k_scale_dh<__bf16>, dim3((unsigned)blocks), dim3(256), 0, st, src, grad_loss, (__bf16*)dH, n);
  else
    hipLaunchKernelGGL(k_scale_dh<float>, dim3((unsigned)blocks), dim3(256), 0, st, src, grad_loss, (float*)dH, n);
  return hipGetLastError();
}

}  // namespace cutbce
