// Preparation kernels of the CutBCE sweeps (all HBM-bound, small next to the sweeps):
//   * row compaction: the list of valid rows, their weights and s = 1 / (W V) from the row mask and weights
//     (padding positions are excluded from the average, "Cut Binary Cross Entropy" Section III-B after
//     Eq. (4)), with no host synchronisation;
//   * H preparation: valid rows gathered into a dense, zero-padded Hc, the slot-packed copy Hrp of the
//     weighted rows (second GEMM operand of the dE sweep) and the weighted column sum of the valid rows;
//   * E preparation: the slot-packed copy Evp (second GEMM operand of the forward/dH sweep) and sum_v E[v];
//   * positive-id buckets: the sparse targets (Listing 1 keeps them as ids, never as a multi-hot Y) grouped
//     by the (tile, step) of each sweep, so a wave finds the positives of its current 32x32 logit tile with
//     two loads;
//   * a multi-block exclusive scan and the target validation kernel.
#include "common.h"

namespace cutbce {

__device__ inline int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

template <typename T> __device__ inline T ld(const T* p) { return *p; }

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

// Exclusive scan of one int per thread over a 1024-thread workgroup; `total` gets the workgroup sum.
__device__ inline int block_excl_scan(int v, int* sh, int& total) {
  // 1024 threads: wave inclusive scan with shuffles, then wave totals through LDS
  const int lane = lane_id(), wave = threadIdx.x / 64;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) off += sh[w];
    tot += sh[w];
  }
  __syncthreads();
  total = tot;
  return off + x - v;
}

// ---------------------------------------------------------------------------------------------------------
// Row compaction in two passes over chunks of 4096 rows (one workgroup each, 4 consecutive rows per thread):
//   count  : the chunk's valid rows and the float64 sum of their weights (each thread adds its rows in order,
//            then a fixed tree over the workgroup);
//   scatter: the chunk's first compact index is the sum of the counts before it; a workgroup scan then places
//            every valid row in ascending order: row_of[k], compact_of[r], rptr[k] (the row's id range clamped
//            into [0, nnz]) and wc[k] = its weight (1 without weights). All chunks clear their share of the
//            padding entries [R_v, R_pad), and chunk 0 writes R_v and s = 1 / (W V), W = the chunk sums added
//            in chunk order.
// ---------------------------------------------------------------------------------------------------------
constexpr int kCompactChunk = 4096;

__device__ inline double block_sum_f64(double x, double* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  if (lane_id() == 0) sh[threadIdx.x / 64] = x;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < 16; ++i) t += sh[i];
  __syncthreads();
  return t;
}

__global__ void __launch_bounds__(1024) k_compact_count(const uint8_t* __restrict__ mask,
                                                        const float* __restrict__ weight, int64_t R,
                                                        int32_t* __restrict__ cnt, double* __restrict__ wsum) {
  __shared__ int sh[16];
  __shared__ double shw[16];
  const int64_t r0 = (int64_t)blockIdx.x * kCompactChunk + 4 * threadIdx.x;
  int n = 0;
  double w = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (r0 + j < R && mask[r0 + j] != 0) {
      ++n;
      w += (double)(weight ? weight[r0 + j] : 1.f);
    }
  int tot;
  (void)block_excl_scan(n, sh, tot);
  const double wt = block_sum_f64(w, shw);
  if (threadIdx.x == 0) {
    cnt[blockIdx.x] = tot;
    wsum[blockIdx.x] = wt;
  }
}

__global__ void __launch_bounds__(1024) k_compact_scatter(const uint8_t* __restrict__ mask,
                                                          const float* __restrict__ weight,
                                                          const int32_t* __restrict__ row_offsets, int64_t R,
                                                          int64_t R_pad, int64_t V, int64_t nnz,
                                                          const int32_t* __restrict__ cnt,
                                                          const double* __restrict__ wsum, Ctl* ctl,
                                                          int32_t* row_of, int32_t* compact_of, int2* rptr,
                                                          float* wc) {
  __shared__ int sh[16];
  const int tid = threadIdx.x;
  const int nchunks = gridDim.x;
  int base = 0, nv = 0;
  for (int b = 0; b < nchunks; ++b) {
    const int c = cnt[b];
    base += b < (int)blockIdx.x ? c : 0;
    nv += c;
  }
  const int64_t r0 = (int64_t)blockIdx.x * kCompactChunk + 4 * tid;
  bool f[4];
  int n = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = r0 + j < R && mask[r0 + j] != 0;
    n += f[j] ? 1 : 0;
  }
  int tot;
  int k = base + block_excl_scan(n, sh, tot);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t r = r0 + j;
    if (r < R) {
      if (f[j]) {
        wc[k] = weight ? weight[r] : 1.f;
        row_of[k] = (int32_t)r;
        compact_of[r] = k;
        // the row's id range, clamped into [0, nnz] (inconsistent offsets give an empty or shortened range)
        const int64_t b = row_offsets[r] < 0 ? 0 : (row_offsets[r] > nnz ? nnz : row_offsets[r]);
        const int64_t e = row_offsets[r + 1] < b ? b : (row_offsets[r + 1] > nnz ? nnz : row_offsets[r + 1]);
        rptr[k] = make_int2((int)b, (int)e);
        ++k;
      } else {
        compact_of[r] = -1;
      }
    }
  }
  for (int64_t q = nv + (int64_t)blockIdx.x * 1024 + tid; q < R_pad; q += (int64_t)nchunks * 1024) {
    row_of[q] = -1;
    rptr[q] = make_int2(0, 0);
    wc[q] = 0.f;
  }
  if (blockIdx.x == 0 && tid == 0) {
    double W = 0.0;
    for (int b = 0; b < nchunks; ++b) W += wsum[b];
    ctl->n_valid = nv;
    ctl->splits = 0;
    ctl->bad_ids = 0;
    ctl->hnorm_max = 0u;
    ctl->hw_absmax = 0u;
    ctl->enorm_max = 0u;
    ctl->e_absmax = 0u;
    ctl->scale = W != 0.0 ? 1.0 / (W * (double)V) : 0.0;
  }
}

hipError_t launch_compact(const Layout& L, char* ws, const uint8_t* mask, const float* weight,
                          const int32_t* row_offsets, hipStream_t st) {
  const int64_t nchunks = (L.R + kCompactChunk - 1) / kCompactChunk;
  double* wsum = (double*)(ws + L.off_cpart);  // [nchunks] doubles, then [nchunks] ints
  int32_t* cnt = (int32_t*)(ws + L.off_cpart + sizeof(double) * nchunks);
  hipLaunchKernelGGL(k_compact_count, dim3((unsigned)nchunks), dim3(1024), 0, st, mask, weight, L.R, cnt, wsum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_compact_scatter, dim3((unsigned)nchunks), dim3(1024), 0, st, mask, weight, row_offsets, L.R,
                     L.R_pad, L.V, L.nnz, (const int32_t*)cnt, (const double*)wsum, (Ctl*)(ws + L.off_ctl),
                     (int32_t*)(ws + L.off_row_of), (int32_t*)(ws + L.off_compact_of), (int2*)(ws + L.off_rptr),
                     (float*)(ws + L.off_wc));
  return hipGetLastError();
}


// One slot-packed run (see slot_off) gathered from a [32][D] tile in LDS.
template <typename T>
__device__ inline void set_run(typename Elem<T>::Op& run, const T* tile, int D, int db, int g, int lane);
template <>
__device__ inline void set_run<__bf16>(bf16x8& run, const __bf16* tile, int D, int db, int g, int lane) {
#pragma unroll
  for (int j = 0; j < 8; ++j) run[j] = tile[acc_pos(g * 8 + j, lane / 32) * D + db * 32 + lane % 32];
}
template <>
__device__ inline void set_run<float>(float& run, const float* tile, int D, int db, int g, int lane) {
  run = tile[acc_pos(g, lane / 32) * D + db * 32 + lane % 32];
}

// The bf16 run as f16 scaled by 2^sh (an exact power of two): the 8 significant bits of each value are kept
// exactly wherever the scaled value is a normal f16 (every value within 2^29 of the largest, which the scale
// brings into [2^14, 2^15)).
__device__ inline void set_run_f16(f16x8& run, const __bf16* tile, int D, int db, int g, int lane, float sc) {
#pragma unroll
  for (int j = 0; j < 8; ++j) run[j] = (_Float16)((float)tile[acc_pos(g * 8 + j, lane / 32) * D + db * 32 + lane % 32] * sc);
}

// The same run with each value times its row's weight w[row] (a weight of 1 leaves it unchanged; others round
// once to the element type).
template <typename T>
__device__ inline void set_run_w(typename Elem<T>::Op& run, const T* tile, const float* w, int D, int db, int g,
                                 int lane);
template <>
__device__ inline void set_run_w<__bf16>(bf16x8& run, const __bf16* tile, const float* w, int D, int db, int g,
                                         int lane) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = acc_pos(g * 8 + j, lane / 32);
    run[j] = (__bf16)((float)tile[row * D + db * 32 + lane % 32] * w[row]);
  }
}
template <>
__device__ inline void set_run_w<float>(float& run, const float* tile, const float* w, int D, int db, int g,
                                        int lane) {
  const int row = acc_pos(g, lane / 32);
  run = tile[row * D + db * 32 + lane % 32] * w[row];
}

// ---------------------------------------------------------------------------------------------------------
// H preparation: block = 32 compacted rows. Hc[k] = H[row_of[k]] (0 for padding), Hrp = slot-packed blocks of
// the weighted rows wc[k] Hc[k] (the B operand of the dE sweep's gradient GEMM, so each row's contribution to
// dE carries its weight), per-block float64 column sums of the weighted rows (the dE sweep's 1/2 sum_r w_r H[r]).
// With `stats`, it also raises ctl->hnorm_max to the largest row norm ||H[r]|| and ctl->hw_absmax to the largest
// |w_r H[r][d]| of the block (unsigned maxima of non-negative float bits, so the result is order-independent).
// ---------------------------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) k_prep_h(const T* __restrict__ H, const int32_t* __restrict__ row_of,
                                                const float* __restrict__ wc, int D, T* __restrict__ Hc,
                                                T* __restrict__ Hrp, double* __restrict__ sum_part,
                                                Ctl* __restrict__ stats, const Ctl* __restrict__ ctl) {
  extern __shared__ char smem_raw[];
  T* tile = (T*)smem_raw;  // [32][D]
  __shared__ float wt[32];
  const int tid = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * 32;
  // no sweep reads compacted rows at or past the valid rows rounded up to a 256-row tile: such blocks only zero
  // their column-sum partials
  if (k0 >= (((int64_t)ctl->n_valid + 255) / 256) * 256) {
    for (int d = tid; d < D; d += 256) sum_part[blockIdx.x * (int64_t)D + d] = 0.0;
    return;
  }
  if (tid < 32) wt[tid] = wc[k0 + tid];
  // gather rows (16-byte units)
  const int upr = D * (int)sizeof(T) / 16;  // 16-byte units per row
  for (int u = tid; u < 32 * upr; u += 256) {
    const int rr = u / upr, c = u % upr;
    const int32_t src = row_of[k0 + rr];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (src >= 0) v = *(const u32x4*)((const char*)H + ((int64_t)src * D) * sizeof(T) + c * 16);
    *(u32x4*)((char*)tile + ((int64_t)rr * D) * sizeof(T) + c * 16) = v;
    *(u32x4*)((char*)Hc + ((k0 + rr) * D) * sizeof(T) + c * 16) = v;
  }
  __syncthreads();
  if (Hrp) {
    T* dst = Hrp + k0 * D;
    const int runs = (D / 32) * Elem<T>::kGroups * 64;
    for (int q = tid; q < runs; q += 256) {
      const int lane = q % 64, g = (q / 64) % Elem<T>::kGroups, db = q / (64 * Elem<T>::kGroups);
      const int64_t o = slot_off<T>(D, db, g, lane);
      typename Elem<T>::Op run;
      set_run_w<T>(run, tile, wt, D, db, g, lane);
      *(typename Elem<T>::Op*)(dst + o) = run;
    }
  }
  for (int d = tid; d < D; d += 256) {
    double s = 0.0;
    for (int rr = 0; rr < 32; ++rr) s += (double)(float)tile[rr * D + d] * (double)wt[rr];
    sum_part[blockIdx.x * (int64_t)D + d] = s;
  }
  if (stats) {
    // 8 lanes per row: squared norm and largest |w x| of the row, then the block maxima
    const int rr = tid / 8, sub = tid % 8;
    float n2 = 0.f, am = 0.f;
    for (int d = sub; d < D; d += 8) {
      const float x = (float)tile[rr * D + d];
      n2 += x * x;
      am = fmaxf(am, fabsf(x * wt[rr]));
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      n2 += __shfl_xor(n2, o, 64);
      am = fmaxf(am, __shfl_xor(am, o, 64));
    }
    float nr = sqrtf(n2);
#pragma unroll
    for (int o = 8; o < 64; o <<= 1) {
      nr = fmaxf(nr, __shfl_xor(nr, o, 64));
      am = fmaxf(am, __shfl_xor(am, o, 64));
    }
    // the block's maxima, then one atomic per field and block
    __shared__ float sh_nr[4], sh_am[4];
    if (lane_id() == 0) {
      sh_nr[tid / 64] = nr;
      sh_am[tid / 64] = am;
    }
    __syncthreads();
    if (tid == 0) {
      atomicMax(&stats->hnorm_max, __float_as_uint(fmaxf(fmaxf(sh_nr[0], sh_nr[1]), fmaxf(sh_nr[2], sh_nr[3]))));
      atomicMax(&stats->hw_absmax, __float_as_uint(fmaxf(fmaxf(sh_am[0], sh_am[1]), fmaxf(sh_am[2], sh_am[3]))));
    }
  }
}

// The slot-packed weighted rows as f16 for the bf16 dE sweep: Hrp = f16(wc[k] Hc[k] 2^s) with
// s = hrp_shift(ctl->hw_absmax) (an exact power of two; the sweep multiplies its sums by 2^-s). Block = 32 rows.
__global__ void __launch_bounds__(256) k_prep_hrp16(const __bf16* __restrict__ Hc, const float* __restrict__ wc,
                                                    const Ctl* __restrict__ ctl, int D, _Float16* __restrict__ Hrp) {
  const int tid = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * 32;
  if (k0 >= (((int64_t)ctl->n_valid + 255) / 256) * 256) return;  // rows no sweep reads (see k_prep_h)
  const int sh = hrp_shift(ctl->hw_absmax);
  _Float16* dst = Hrp + k0 * D;
  if (narrow_owner(1, D)) {
    // the 16-owner engine's layout (D >= 256)
    for (int q = tid; q < (D / 16) * 64; q += 256) {
      const int lane = q % 64, db = q / 64;
      f16x8 run;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = sp16_row(lane, j);
        run[j] = (_Float16)ldexpf((float)Hc[(k0 + row) * D + db * 16 + lane % 16] * wc[k0 + row], sh);
      }
      *(f16x8*)(dst + sp16_off(db, lane)) = run;
    }
    return;
  }
  const int runs = (D / 32) * 2 * 64;
  for (int q = tid; q < runs; q += 256) {
    const int lane = q % 64, g = (q / 64) % 2, db = q / 128;
    f16x8 run;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = acc_pos(g * 8 + j, lane / 32);
      run[j] = (_Float16)ldexpf((float)Hc[(k0 + row) * D + db * 32 + lane % 32] * wc[k0 + row], sh);
    }
    *(f16x8*)(dst + slot_off<__bf16>(D, db, g, lane)) = run;
  }
}

// Column sums of `nparts` rows of float64 partials [nparts][D], in a fixed order, in one or two passes. The
// parts form G groups of `per` consecutive parts (G from nparts alone: one group per 512 parts, at most
// kSumMaxGroups). Pass 1, block (x, g): 16 columns x 64 part lanes; lane y adds parts y, y + 64, ... of group g
// into four running sums (m mod 4, so four loads are in flight), adds those four, and the 64 lane sums of a
// column are added in order of y. With one group that is the result; otherwise pass 2 adds the G group sums of
// each column in group order.
constexpr int kSumCols = 16, kSumLanes = 64, kSumPartsPerGroup = 512;

__global__ void __launch_bounds__(1024) k_sum_parts(const double* __restrict__ part, int64_t nparts, int D,
                                                    int64_t per, double* __restrict__ out) {
  __shared__ double sh[kSumLanes][kSumCols + 1];
  const int c = threadIdx.x % kSumCols, y = threadIdx.x / kSumCols;
  const int d = blockIdx.x * kSumCols + c;
  const int64_t p0 = (int64_t)blockIdx.y * per;
  const int64_t p1 = p0 + per < nparts ? p0 + per : nparts;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  if (d < D) {
    int64_t p = p0 + y;
    for (; p + 3 * kSumLanes < p1; p += 4 * kSumLanes) {
#pragma unroll
      for (int q = 0; q < 4; ++q) s[q] += part[(p + q * kSumLanes) * D + d];
    }
    // at most three parts are left
    if (p < p1) s[0] += part[p * D + d];
    if (p + kSumLanes < p1) s[1] += part[(p + kSumLanes) * D + d];
    if (p + 2 * kSumLanes < p1) s[2] += part[(p + 2 * kSumLanes) * D + d];
  }
  sh[y][c] = (s[0] + s[1]) + (s[2] + s[3]);
  __syncthreads();
  if (y == 0 && d < D) {
    double t = 0.0;
    for (int yy = 0; yy < kSumLanes; ++yy) t += sh[yy][c];
    out[(int64_t)blockIdx.y * D + d] = t;
  }
}

__global__ void k_sum_groups(const double* __restrict__ gsum, int G, int D, double* __restrict__ out) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  if (d >= D) return;
  double t = 0.0;
  for (int g0 = 0; g0 < G; g0 += 8) {  // eight loads in flight, added in group order
    double x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = gsum[(int64_t)min(g0 + j, G - 1) * D + d];  // past G: unused
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (g0 + j < G) t += x[j];
  }
  out[d] = t;
}

static hipError_t sum_parts(const Layout& L, char* ws, const double* part, int64_t nparts, double* out,
                            hipStream_t st) {
  int64_t G = (nparts + kSumPartsPerGroup - 1) / kSumPartsPerGroup;
  G = G < 1 ? 1 : (G > kSumMaxGroups ? kSumMaxGroups : G);
  const int64_t per = (nparts + G - 1) / G;
  double* gsum = (double*)(ws + L.off_sum2);  // [G][D] group sums
  hipLaunchKernelGGL(k_sum_parts, dim3((unsigned)((L.D + kSumCols - 1) / kSumCols), (unsigned)G), dim3(1024), 0, st,
                     part, nparts, L.D, per, G == 1 ? out : gsum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || G == 1) return e;
  hipLaunchKernelGGL(k_sum_groups, dim3((unsigned)((L.D + 255) / 256)), dim3(256), 0, st, (const double*)gsum, (int)G,
                     L.D, out);
  return hipGetLastError();
}

hipError_t launch_prep_h(const Layout& L, char* ws, const void* H, bool want_hrp, hipStream_t st) {
  const int64_t nblk = L.R_pad / 32;
  const size_t sm = (size_t)32 * L.D * L.esz;
  // the f16 copy for the bf16 dE sweep is written by a second kernel once the scale is known
  const bool f16rp = want_hrp && hrp_is_f16(L.dtype, L.D);
  Ctl* ctl = (Ctl*)(ws + L.off_ctl);
  if (L.dtype == 1) {
    // bf16 always takes the row statistics, so that a backward can reuse this preparation (launch_prep_hrp)
    hipLaunchKernelGGL(k_prep_h<__bf16>, dim3((unsigned)nblk), dim3(256), sm, st, (const __bf16*)H,
                       (const int32_t*)(ws + L.off_row_of), (const float*)(ws + L.off_wc), L.D,
                       (__bf16*)(ws + L.off_Hc), want_hrp && !f16rp ? (__bf16*)(ws + L.off_Hrp) : nullptr,
                       (double*)(ws + L.off_sumH_part), ctl, (const Ctl*)ctl);
  } else {
    hipLaunchKernelGGL(k_prep_h<float>, dim3((unsigned)nblk), dim3(256), sm, st, (const float*)H,
                       (const int32_t*)(ws + L.off_row_of), (const float*)(ws + L.off_wc), L.D,
                       (float*)(ws + L.off_Hc),
                       want_hrp ? (float*)(ws + L.off_Hrp) : nullptr, (double*)(ws + L.off_sumH_part), nullptr,
                       (const Ctl*)ctl);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (f16rp && (e = launch_prep_hrp(L, ws, H, st)) != hipSuccess) return e;
  return sum_parts(L, ws, (const double*)(ws + L.off_sumH_part), nblk, (double*)(ws + L.off_sumH), st);
}

hipError_t launch_prep_hrp(const Layout& L, char* ws, const void* H, hipStream_t st) {
  if (!hrp_is_f16(L.dtype, L.D)) return launch_prep_h(L, ws, H, true, st);  // f32: the copy comes from H
  hipLaunchKernelGGL(k_prep_hrp16, dim3((unsigned)(L.R_pad / 32)), dim3(256), 0, st, (const __bf16*)(ws + L.off_Hc),
                     (const float*)(ws + L.off_wc), (const Ctl*)(ws + L.off_ctl), L.D, (_Float16*)(ws + L.off_Hrp));
  return hipGetLastError();
}

// E statistics of the f16-Evp shapes (bf16, D <= 128): one block folds the E preparation blocks' maxima
// (max ||E[v]||, max |E|; NaNs do not enter them, and a NaN in E gives NaN outputs on either forward epilogue)
// into the control block, and decides whether the shift Evp was written with stands: it must put max |E| in
// [2^13, 2^15) (no f16 overflow; 11 significant bits for every value within 2^27 of the largest). Otherwise it
// records the shift that puts max |E| in [2^14, 2^15) and sets evp_fix, and the fix-up pass of k_prep_e rewrites
// Evp. (Scaling from statistics of a separate pass over E before the preparation cost one more read of E,
// 45 us at 876,000 x 128.)
__global__ void __launch_bounds__(1024) k_stats_e_final(const float* __restrict__ part, int64_t nblk,
                                                        Ctl* __restrict__ ctl) {
  __shared__ float sh[2][16];
  const int tid = threadIdx.x;
  float n = 0.f, a = 0.f;
  for (int64_t b = tid; b < nblk; b += 1024) {
    n = fmaxf(n, part[2 * b]);
    a = fmaxf(a, part[2 * b + 1]);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    n = fmaxf(n, __shfl_xor(n, o, 64));
    a = fmaxf(a, __shfl_xor(a, o, 64));
  }
  if (tid % 64 == 0) {
    sh[0][tid / 64] = n;
    sh[1][tid / 64] = a;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 16; ++w) {
      n = fmaxf(n, sh[0][w]);
      a = fmaxf(a, sh[1][w]);
    }
    ctl->enorm_max = __float_as_uint(n);
    ctl->e_absmax = __float_as_uint(a);
    const int used = evp_shift_of(ctl), want = hrp_shift(__float_as_uint(a));
    const bool fix = !(used == want || used == want - 1);
    ctl->evp_fix = fix ? 1 : 0;
    if (fix) ctl->evp_shift = want;
  }
}

// ---------------------------------------------------------------------------------------------------------
// E preparation: block = kEBlkItems items, processed 32 at a time through LDS. Writes the slot-packed Evp
// (when requested; f16 scaled by 2^evp_shift for the evp_is_f16 shapes) and float64 column sums per block; for
// the f16-Evp shapes also the block's max ||E[v]|| and max |E| (stat[2 b], stat[2 b + 1]). FIX: the fix-up pass
// (launched after k_stats_e_final): every block returns at once unless evp_fix is set, and then only rewrites
// Evp with the new shift.
// ---------------------------------------------------------------------------------------------------------
template <typename T, int D, bool FIX = false>
__global__ void __launch_bounds__(256) k_prep_e(const T* __restrict__ E, int64_t V, T* __restrict__ Evp,
                                                double* __restrict__ sum_part, const Ctl* __restrict__ ctl,
                                                float* __restrict__ stat) {
  extern __shared__ char smem_raw[];
  T* tile = (T*)smem_raw;  // [32][D]
  const int tid = threadIdx.x;
  if (FIX && ctl->evp_fix == 0) return;  // block-uniform
  constexpr bool kStats = sizeof(T) == 2 && evp_is_f16(1, D) && !FIX;
  float nmax = 0.f, amax = 0.f;  // kStats: this thread's largest item norm^2 and |value| so far
  constexpr int upr = D * (int)sizeof(T) / 16;  // 16-byte units per row
  constexpr int kU = 32 * upr / 256;             // units per thread and 32-item chunk (1 ... 8)
  static_assert(kU >= 1 && 32 * upr % 256 == 0, "whole units per thread");
  double acc0 = 0.0, acc1 = 0.0;  // column sums for d = tid and d = tid + 256
  const int64_t v_begin = (int64_t)blockIdx.x * kEBlkItems;
  // unit u = tid + 256 q of a chunk; the next chunk's units are loaded while the current one is packed
  u32x4 nx[kU];
  auto load_chunk = [&](int64_t v0) {
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int u = tid + 256 * q, rr = u / upr, c = u % upr;
      nx[q] = u32x4{0u, 0u, 0u, 0u};
      if (v0 + rr < V) nx[q] = *(const u32x4*)((const char*)E + ((v0 + rr) * D) * sizeof(T) + c * 16);
    }
  };
  load_chunk(v_begin);
  for (int ch = 0; ch < kEBlkItems / 32; ++ch) {
    const int64_t v0 = v_begin + ch * 32;
#pragma unroll
    for (int q = 0; q < kU; ++q) {
      const int u = tid + 256 * q, rr = u / upr, c = u % upr;
      *(u32x4*)((char*)tile + ((int64_t)rr * D) * sizeof(T) + c * 16) = nx[q];
    }
    __syncthreads();
    if (ch + 1 < kEBlkItems / 32) load_chunk(v0 + 32);
    bool packed = false;
    if constexpr (sizeof(T) == 2) {
      if (Evp && narrow_owner(1, D)) {
        // the 16-owner engine's layout (bf16, D >= 256)
        T* dst = Evp + v0 * D;
        for (int q = tid; q < (D / 16) * 64; q += 256) {
          const int lane = q % 64, db = q / 64;
          bf16x8 run;
#pragma unroll
          for (int j = 0; j < 8; ++j) run[j] = tile[sp16_row(lane, j) * D + db * 16 + lane % 16];
          *(bf16x8*)(dst + sp16_off(db, lane)) = run;
        }
        packed = true;
      }
    }
    if constexpr (kStats) {
      if (stat) {
        // 8 threads per item of the chunk (padding items are zero)
        const int it = tid / 8, sub = tid % 8;
        float n2 = 0.f;
#pragma unroll
        for (int k = 0; k < D / 8; ++k) {
          const float x = (float)tile[it * D + sub + 8 * k];
          n2 += x * x;
          amax = fmaxf(amax, __builtin_fabsf(x));
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) n2 += __shfl_xor(n2, o, 64);
        nmax = fmaxf(nmax, n2);
      }
    }
    if constexpr (sizeof(T) == 2 && evp_is_f16(1, D)) {
      if (Evp) {
        _Float16* dst = (_Float16*)(Evp + v0 * D);
        const float sc = ldexpf(1.f, evp_shift_of(ctl));
        for (int q = tid; q < (D / 32) * 2 * 64; q += 256) {
          const int lane = q % 64, g = (q / 64) % 2, db = q / 128;
          f16x8 run;
          set_run_f16(run, tile, D, db, g, lane, sc);
          *(f16x8*)(dst + slot_off<T>(D, db, g, lane)) = run;
        }
        packed = true;
      }
    }
    if (Evp && !packed) {
      T* dst = Evp + v0 * D;
      const int runs = (D / 32) * Elem<T>::kGroups * 64;
      for (int q = tid; q < runs; q += 256) {
        const int lane = q % 64, g = (q / 64) % Elem<T>::kGroups, db = q / (64 * Elem<T>::kGroups);
        const int64_t o = slot_off<T>(D, db, g, lane);
        typename Elem<T>::Op run;  // kEPL consecutive elements: one 16-byte (bf16) or 4-byte (f32) store
        set_run<T>(run, tile, D, db, g, lane);
        *(typename Elem<T>::Op*)(dst + o) = run;
      }
    }
    if (!FIX) {
      if (tid < D)
        for (int rr = 0; rr < 32; ++rr) acc0 += (double)(float)tile[rr * D + tid];
      if (tid + 256 < D)
        for (int rr = 0; rr < 32; ++rr) acc1 += (double)(float)tile[rr * D + tid + 256];
    }
    __syncthreads();
  }
  if (FIX) return;
  if (tid < D) sum_part[blockIdx.x * (int64_t)D + tid] = acc0;
  if (tid + 256 < D) sum_part[blockIdx.x * (int64_t)D + tid + 256] = acc1;
  if constexpr (kStats) {
    if (stat) {
      __shared__ float sh_n[4], sh_a[4];
#pragma unroll
      for (int o = 8; o < 64; o <<= 1) nmax = fmaxf(nmax, __shfl_xor(nmax, o, 64));
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      if (tid % 64 == 0) {
        sh_n[tid / 64] = nmax;
        sh_a[tid / 64] = amax;
      }
      __syncthreads();
      if (tid == 0) {
        stat[2 * blockIdx.x] = sqrtf(fmaxf(fmaxf(sh_n[0], sh_n[1]), fmaxf(sh_n[2], sh_n[3])));
        stat[2 * blockIdx.x + 1] = fmaxf(fmaxf(sh_a[0], sh_a[1]), fmaxf(sh_a[2], sh_a[3]));
      }
    }
  }
}

template <typename T, int D>
static void prep_e_launch(const Layout& L, char* ws, const void* E, bool want_evp, hipStream_t st) {
  Ctl* ctl = (Ctl*)(ws + L.off_ctl);
  constexpr bool kF16 = sizeof(T) == 2 && evp_is_f16(1, D);
  float* stat = kF16 && want_evp ? (float*)(ws + L.off_estat) : nullptr;
  T* evp = want_evp ? (T*)(ws + L.off_Evp) : nullptr;
  const size_t sm = (size_t)32 * D * sizeof(T);
  hipLaunchKernelGGL((k_prep_e<T, D>), dim3((unsigned)L.n_eblk), dim3(256), sm, st, (const T*)E, L.V, evp,
                     (double*)(ws + L.off_sumE_part), (const Ctl*)ctl, stat);
  if (stat) {
    hipLaunchKernelGGL(k_stats_e_final, dim3(1), dim3(1024), 0, st, (const float*)stat, L.n_eblk, ctl);
    hipLaunchKernelGGL((k_prep_e<T, D, true>), dim3((unsigned)L.n_eblk), dim3(256), sm, st, (const T*)E, L.V, evp,
                       (double*)nullptr, (const Ctl*)ctl, (float*)nullptr);
  }
}

hipError_t launch_prep_e(const Layout& L, char* ws, const void* E, bool want_evp, hipStream_t st) {
  if (L.dtype == 1) {
    switch (L.D) {
      case 64: prep_e_launch<__bf16, 64>(L, ws, E, want_evp, st); break;
      case 128: prep_e_launch<__bf16, 128>(L, ws, E, want_evp, st); break;
      case 256: prep_e_launch<__bf16, 256>(L, ws, E, want_evp, st); break;
      case 512: prep_e_launch<__bf16, 512>(L, ws, E, want_evp, st); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (L.D) {
      case 64: prep_e_launch<float, 64>(L, ws, E, want_evp, st); break;
      case 128: prep_e_launch<float, 128>(L, ws, E, want_evp, st); break;
      case 256: prep_e_launch<float, 256>(L, ws, E, want_evp, st); break;
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return sum_parts(L, ws, (const double*)(ws + L.off_sumE_part), L.n_eblk, (double*)(ws + L.off_sumE), st);
}

// ---------------------------------------------------------------------------------------------------------
// Multi-block exclusive scan of int32 counts, in place: x[i] <- sum_{j<i} x[j] for i <= n (x[n] = total), and
// optionally the scanned x[0..n) copied to `copy` as well. Thread t of block b owns the 8 entries from
// b * kScanBlock + 8 t (one 32-byte run: two 16-byte loads and stores where the run lies inside [0, n)); entry n
// (the grand total) falls in the first run that reaches past n - 1. Two passes: k_scan_sums leaves each block's
// total; k_scan_apply adds up the totals of the blocks before its own, then scans its block.
// ---------------------------------------------------------------------------------------------------------
constexpr int kScanPerThread = kScanBlock / 1024;
static_assert(kScanPerThread == 8, "two 16-byte vectors per thread");

__device__ inline void scan_load8(const int32_t* __restrict__ x, int64_t b0, int64_t n, int* v) {
  if (b0 + 8 <= n) {
    const int4 a = *(const int4*)(x + b0), b = *(const int4*)(x + b0 + 4);
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = b0 + j < n ? x[b0 + j] : 0;
  }
}

__global__ void __launch_bounds__(1024) k_scan_sums(const int32_t* __restrict__ x, int64_t n,
                                                    int32_t* __restrict__ bsum) {
  __shared__ int sh[16];
  const int64_t b0 = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * kScanPerThread;
  int v[8];
  scan_load8(x, b0, n, v);
  int s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += v[j];
  int tot;
  block_excl_scan(s, sh, tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

__global__ void __launch_bounds__(1024) k_scan_apply(int32_t* __restrict__ x, int64_t n,
                                                     const int32_t* __restrict__ bsum, int32_t* __restrict__ copy) {
  __shared__ int sh[16];
  const int64_t b0 = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * kScanPerThread;
  int v[8];
  scan_load8(x, b0, n, v);
  int s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += v[j];
  // the block's base: the sums of the blocks before it (integers: any order gives the same total)
  int before = 0;
  for (int64_t i = threadIdx.x; i < (int64_t)blockIdx.x; i += 1024) before += bsum[i];
  int base, tot;
  (void)block_excl_scan(before, sh, base);
  int run = block_excl_scan(s, sh, tot) + base;
  int o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    o[j] = run;
    run += v[j];
  }
  if (b0 + 8 <= n) {
    const int4 a = make_int4(o[0], o[1], o[2], o[3]), b = make_int4(o[4], o[5], o[6], o[7]);
    *(int4*)(x + b0) = a;
    *(int4*)(x + b0 + 4) = b;
    if (copy) {
      *(int4*)(copy + b0) = a;
      *(int4*)(copy + b0 + 4) = b;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (b0 + j <= n) x[b0 + j] = o[j];  // entry n receives the grand total
      if (copy && b0 + j < n) copy[b0 + j] = o[j];
    }
  }
}

static hipError_t scan_exclusive(int32_t* x, int64_t n, int32_t* tmp, int32_t* copy, hipStream_t st) {
  // n + 1 entries are written; blocks cover [0, n] inclusive
  const int64_t nb = (n + 1 + kScanBlock - 1) / kScanBlock;
  hipLaunchKernelGGL(k_scan_sums, dim3((unsigned)nb), dim3(1024), 0, st, x, n, tmp);
  hipLaunchKernelGGL(k_scan_apply, dim3((unsigned)nb), dim3(1024), 0, st, x, n, (const int32_t*)tmp, copy);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------------
// Positive-id buckets. Pairs (compact row k, item v) go to
//   rows side : bucket (k / rows_per_wg) * n_vs + v / 32      (forward sweep: row tile x item step)
//   items side: bucket (v / items_per_wg) * n_rs + k / 32     (backward sweep: item tile x row step)
// Ids outside [0, V) are skipped and counted. Order inside a bucket is irrelevant: the sweeps OR the
// positives into a per-lane bit mask, which also makes a repeated id count once.
// Two forms, chosen from the mean row length:
//  - k_bucket: 8 lanes per row, one atomic per id (rows holding a handful of ids);
//  - k_bucket_runs: one wave per row, 64 ids at a time. Consecutive lanes whose ids fall in the same bucket
//    (sorted ids of a long row mostly do) form a run; the run's first lane reserves the whole run with one
//    atomic and the others take the following slots. With many ids per row and hot items, one atomic per id
//    serialises on the hot buckets' counters.
// ---------------------------------------------------------------------------------------------------------
// Wave-aggregated counter increments: the active lanes that target one bucket make a single atomic (issued by
// the first of them), and each gets base + its rank among them. Many lanes of a wave hit the same bucket when
// items are hot (a Zipf head in one item tile), where one atomic per id would serialise on that counter.
// Uniform control flow: every lane of the wave must call it.
__device__ inline int aggregated_add(int32_t* __restrict__ cnt, int64_t b, bool active) {
  const int lane = lane_id();
  uint64_t todo = __ballot(active);
  int slot = 0;
  while (todo) {
    const int leader = __builtin_ctzll(todo);
    const int64_t bl = __shfl(b, leader, 64);
    const uint64_t m = __ballot(active && b == bl) & todo;
    int base = 0;
    if (lane == leader) base = atomicAdd(&cnt[bl], __popcll(m));
    base = __shfl(base, leader, 64);
    if ((m >> lane) & 1) slot = base + __popcll(m & ((1ull << lane) - 1));
    todo &= ~m;
  }
  return slot;
}

// A compacted row's id range [x, y) clamped into [0, nnz] (the compaction already clamps it; clamping again keeps
// the reads inside item_ids whatever the workspace holds).
__device__ inline int2 clamp_range(int2 r, int64_t nnz) {
  const int n = (int)nnz;
  const int b = min(max(r.x, 0), n);
  return make_int2(b, min(max(r.y, b), n));
}

template <bool kScatter>
__global__ void __launch_bounds__(256) k_bucket(const Ctl* __restrict__ ctl, const int2* __restrict__ rptr,
                                                const int32_t* __restrict__ ids, int64_t V, int64_t nnz,
                                                bool rows_side, int tile, int64_t nsteps_minor,
                                                int32_t* __restrict__ cnt, int2* __restrict__ pairs, int* bad) {
  const int64_t k = (int64_t)blockIdx.x * (blockDim.x / 8) + threadIdx.x / 8;
  const int sub = threadIdx.x % 8;
  const bool row = k < ctl->n_valid;
  const int2 rp = row ? clamp_range(rptr[k], nnz) : make_int2(0, 0);
  // the wave's longest row sets the (uniform) number of rounds
  int len = rp.y - rp.x;
#pragma unroll
  for (int o = 8; o < 64; o <<= 1) len = max(len, __shfl_xor(len, o, 64));
  int nbad = 0;
  for (int p0 = 0; p0 < len; p0 += 8) {
    const int p = rp.x + p0 + sub;
    bool act = p < rp.y;
    int v = 0;
    if (act) {
      v = ids[p];
      if (v < 0 || v >= V) {
        ++nbad;
        act = false;
      }
    }
    const int64_t b = rows_side ? (k / tile) * nsteps_minor + v / 32 : ((int64_t)v / tile) * nsteps_minor + k / 32;
    const int pos = aggregated_add(cnt, b, act);
    if (kScatter && act) pairs[pos] = make_int2((int)k, v);
  }
  if (!kScatter && nbad) atomicAdd(bad, nbad);
}

template <bool kScatter>
__global__ void __launch_bounds__(256) k_bucket_runs(const Ctl* __restrict__ ctl, const int2* __restrict__ rptr,
                                                     const int32_t* __restrict__ ids, int64_t V, int64_t nnz,
                                                     bool rows_side, int tile, int64_t nsteps_minor,
                                                     int32_t* __restrict__ cnt, int2* __restrict__ pairs, int* bad) {
  const int64_t k = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;  // one row per wave
  const int lane = lane_id();
  if (k >= ctl->n_valid) return;  // the whole wave
  const int2 rp = clamp_range(rptr[k], nnz);
  int nbad = 0;
  for (int p0 = rp.x; p0 < rp.y; p0 += 64) {  // uniform across the wave
    const int p = p0 + lane;
    long long b = -1;  // bucket, or -1 past the row's end and for ids outside [0, V)
    int v = 0;
    if (p < rp.y) {
      v = ids[p];
      if (v < 0 || v >= V)
        ++nbad;
      else
        b = rows_side ? (k / tile) * nsteps_minor + v / 32 : (v / tile) * nsteps_minor + k / 32;
    }
    // a run starts at lane 0 and wherever the bucket differs from the previous lane's
    const long long prev = __shfl_up(b, 1, 64);
    const unsigned long long starts = __ballot(lane == 0 || b != prev);
    const unsigned long long upto = lane == 63 ? ~0ull : ((2ull << lane) - 1);  // lanes 0..lane
    const int head = 63 - __clzll(starts & upto);                               // lane 0 is always a start
    const unsigned long long after = starts & ~upto;
    const int end = after ? __ffsll((long long)after) - 1 : 64;
    int base = 0;
    if (b >= 0 && lane == head) base = atomicAdd(&cnt[b], end - head);
    if (kScatter) {
      base = __shfl(base, head, 64);
      if (b >= 0) pairs[base + (lane - head)] = make_int2((int)k, v);
    }
  }
  if (!kScatter) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) nbad += __shfl_xor(nbad, o, 64);
    if (lane == 0 && nbad) atomicAdd(bad, nbad);
  }
}

hipError_t launch_buckets(const Layout& L, char* ws, const int32_t* item_ids, bool rows_side, hipStream_t st) {
  const int64_t nb = rows_side ? L.nb_r : L.nb_i;
  int32_t* bptr = (int32_t*)(ws + (rows_side ? L.off_bptr_r : L.off_bptr_i));
  int32_t* bfill = (int32_t*)(ws + (rows_side ? L.off_bfill_r : L.off_bfill_i));
  int2* pairs = (int2*)(ws + (rows_side ? L.off_pairs_r : L.off_pairs_i));
  Ctl* ctl = (Ctl*)(ws + L.off_ctl);
  const int tile = rows_side ? L.rows_per_wg : L.items_per_wg;
  const int64_t minor = rows_side ? L.n_vs : L.n_rs;
  hipError_t e = launch_fill_i32(bptr, nb + 1, 0, st);
  if (e != hipSuccess) return e;
  // wave-per-row runs when rows average more than 32 ids (host-side sizes only)
  const bool runs = L.nnz > 32 * L.R;
  const int64_t blocks = runs ? L.R_pad / 4 : L.R_pad / 32;  // rows per 256-thread block: 4 or 32
  if (L.nnz > 0) {
    hipLaunchKernelGGL(runs ? k_bucket_runs<false> : k_bucket<false>, dim3((unsigned)blocks), dim3(256), 0, st,
                       ctl, (const int2*)(ws + L.off_rptr), item_ids, L.V, L.nnz, rows_side, tile, minor, bptr,
                       (int2*)nullptr, &ctl->bad_ids);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the scan also leaves the bucket starts in bfill, the scatter's running counters
  if ((e = scan_exclusive(bptr, nb, (int32_t*)(ws + L.off_scan), L.nnz > 0 ? bfill : nullptr, st)) != hipSuccess)
    return e;
  if (L.nnz > 0) {
    hipLaunchKernelGGL(runs ? k_bucket_runs<true> : k_bucket<true>, dim3((unsigned)blocks), dim3(256), 0, st,
                       ctl, (const int2*)(ws + L.off_rptr), item_ids, L.V, L.nnz, rows_side, tile, minor, bfill, pairs,
                       (int*)nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_no_row_buckets(const Layout& L, char* ws, hipStream_t st) {
  // the bf16 forward sweeps without Cut Metrics are compiled without positives and read no bucket pointers
  if (L.dtype == 1) return hipSuccess;
  return launch_fill_i32((int32_t*)(ws + L.off_bptr_r), L.nb_r + 1, 0, st);
}

// ---------------------------------------------------------------------------------------------------------
// Dense padded targets -> CSR ("Cut Binary Cross Entropy", Listing 1 takes targets as [B, N, L] id slots).
// Row r's ids are targets[r][0..L) in slot order with every slot equal to pad_id dropped.
//   count  : row_offsets[r + 1] = number of kept slots of row r; row_offsets[0] = 0
//   scan   : one workgroup turns row_offsets[1..R] into inclusive prefix sums, 1024 rows at a time
//   scatter: row r writes its kept ids, in slot order, to item_ids[row_offsets[r]...]
// ---------------------------------------------------------------------------------------------------------
__global__ void k_t2c_count(const int32_t* __restrict__ targets, int64_t R, int L, int32_t pad,
                            int32_t* __restrict__ row_offsets) {
  const int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (r == 0) row_offsets[0] = 0;
  if (r >= R) return;
  int n = 0;
  for (int k = 0; k < L; ++k) n += targets[r * L + k] != pad ? 1 : 0;
  row_offsets[r + 1] = n;
}

__global__ void __launch_bounds__(1024) k_t2c_scan(int32_t* __restrict__ x, int64_t n) {
  __shared__ int sh[16];
  int base = 0;
  for (int64_t c0 = 0; c0 < n; c0 += 1024) {
    const int64_t i = c0 + threadIdx.x;
    const int v = i < n ? x[i] : 0;
    int tot;
    const int ex = block_excl_scan(v, sh, tot);
    if (i < n) x[i] = base + ex + v;
    base += tot;
  }
}

__global__ void k_t2c_scatter(const int32_t* __restrict__ targets, int64_t R, int L, int32_t pad,
                              const int32_t* __restrict__ row_offsets, int32_t* __restrict__ item_ids) {
  const int64_t r = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (r >= R) return;
  int o = row_offsets[r];
  for (int k = 0; k < L; ++k) {
    const int32_t v = targets[r * L + k];
    if (v != pad) item_ids[o++] = v;
  }
}

hipError_t launch_targets_to_csr(int64_t R, int L, const int32_t* targets, int32_t pad, int32_t* row_offsets,
                                 int32_t* item_ids, hipStream_t st) {
  const unsigned blocks = (unsigned)((R + 255) / 256);
  hipLaunchKernelGGL(k_t2c_count, dim3(blocks), dim3(256), 0, st, targets, R, L, pad, row_offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_t2c_scan, dim3(1), dim3(1024), 0, st, row_offsets + 1, R);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_t2c_scatter, dim3(blocks), dim3(256), 0, st, targets, R, L, pad, row_offsets, item_ids);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------------
// Target validation.
// ---------------------------------------------------------------------------------------------------------
__global__ void k_validate(int64_t R, int64_t V, int64_t nnz, const int32_t* __restrict__ ro,
                           const int32_t* __restrict__ ids, int32_t* bad) {
  int nb = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  for (int64_t r = t0; r < R; r += stride)
    if (ro[r + 1] < ro[r]) ++nb;
  const int64_t used = ro[R] < nnz ? (ro[R] > 0 ? ro[R] : 0) : nnz;  // ids past row_offsets[R] are unused
  for (int64_t p = t0; p < used; p += stride)
    if (ids[p] < 0 || ids[p] >= V) ++nb;
  if (t0 == 0 && (ro[0] != 0 || ro[R] > nnz)) ++nb;
  if (nb) atomicAdd(bad, nb);
}

hipError_t launch_validate(int64_t R, int64_t V, int64_t nnz, const int32_t* row_offsets,
                           const int32_t* item_ids, int32_t* bad, hipStream_t st) {
  hipError_t e = launch_fill_i32(bad, 1, 0, st);
  if (e != hipSuccess) return e;
  int64_t n = R > nnz ? R : nnz;
  int64_t blocks = (n + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_validate, dim3((unsigned)blocks), dim3(256), 0, st, R, V, nnz, row_offsets, item_ids, bad);
  return hipGetLastError();
}

}  // namespace cutbce
