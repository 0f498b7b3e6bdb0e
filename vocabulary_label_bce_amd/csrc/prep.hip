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

// Plain int copy as a kernel (a kernel node when the caller captures the stream into a graph).
__global__ void k_copy_i32(int32_t* __restrict__ dst, const int32_t* __restrict__ src, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
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
// Row compaction: one workgroup walks the mask in chunks of 4096 rows (4 consecutive rows per thread), keeping
// ascending order. Each valid row's weight (1 without weights) goes to wc[k]; their sum W, in float64 (each
// thread adds its rows in order, then the 1024 partial sums are added in a fixed tree), gives s = 1 / (W V).
// ---------------------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) k_compact(const uint8_t* __restrict__ mask,
                                                  const float* __restrict__ weight,
                                                  const int32_t* __restrict__ row_offsets, int64_t R,
                                                  int64_t R_pad, int64_t V, int64_t nnz, Ctl* ctl,
                                                  int32_t* row_of, int32_t* compact_of, int2* rptr, float* wc) {
  __shared__ int sh[16];
  __shared__ double shw[16];
  const int tid = threadIdx.x;
  int base = 0;
  double wsum = 0.0;
  for (int64_t c0 = 0; c0 < R; c0 += 4096) {
    const int64_t r0 = c0 + 4 * tid;
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
          const float w = weight ? weight[r] : 1.f;
          wsum += (double)w;
          wc[k] = w;
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
    base += tot;
  }
  const int nv = base;
  for (int64_t k = nv + tid; k < R_pad; k += 1024) {
    row_of[k] = -1;
    rptr[k] = make_int2(0, 0);
    wc[k] = 0.f;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o, 64);
  if (lane_id() == 0) shw[tid / 64] = wsum;
  __syncthreads();
  if (tid == 0) {
    double W = 0.0;
    for (int i = 0; i < 16; ++i) W += shw[i];
    ctl->n_valid = nv;
    ctl->splits = 0;
    ctl->bad_ids = 0;
    ctl->scale = W != 0.0 ? 1.0 / (W * (double)V) : 0.0;
  }
}

hipError_t launch_compact(const Layout& L, char* ws, const uint8_t* mask, const float* weight,
                          const int32_t* row_offsets, hipStream_t st) {
  hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, st, mask, weight, row_offsets, L.R, L.R_pad, L.V, L.nnz,
                     (Ctl*)(ws + L.off_ctl), (int32_t*)(ws + L.off_row_of), (int32_t*)(ws + L.off_compact_of),
                     (int2*)(ws + L.off_rptr), (float*)(ws + L.off_wc));
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
// ---------------------------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) k_prep_h(const T* __restrict__ H, const int32_t* __restrict__ row_of,
                                                const float* __restrict__ wc, int D, T* __restrict__ Hc,
                                                T* __restrict__ Hrp, double* __restrict__ sum_part) {
  extern __shared__ char smem_raw[];
  T* tile = (T*)smem_raw;  // [32][D]
  __shared__ float wt[32];
  const int tid = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * 32;
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
}

// Sum `nparts` rows of float64 partials [nparts][D] in a fixed order: block = 32 columns x 32 part lanes; part
// lane y adds parts y + 32 m for m = 0, 1, ... into four running sums (m mod 4, so four loads are in flight),
// adds those four, then the 32 lane sums are added in order of y.
__global__ void __launch_bounds__(1024) k_sum_parts(const double* __restrict__ part, int64_t nparts, int D,
                                                    double* __restrict__ out) {
  __shared__ double sh[32][33];
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;
  const int d = blockIdx.x * 32 + tx;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  if (d < D) {
    int64_t p = ty;
    for (; p + 96 < nparts; p += 128) {
#pragma unroll
      for (int q = 0; q < 4; ++q) s[q] += part[(p + 32 * q) * D + d];
    }
    // at most three parts are left
    if (p < nparts) s[0] += part[p * D + d];
    if (p + 32 < nparts) s[1] += part[(p + 32) * D + d];
    if (p + 64 < nparts) s[2] += part[(p + 64) * D + d];
  }
  sh[ty][tx] = (s[0] + s[1]) + (s[2] + s[3]);
  __syncthreads();
  if (ty == 0 && d < D) {
    double t = 0.0;
    for (int y = 0; y < 32; ++y) t += sh[y][tx];
    out[d] = t;
  }
}

hipError_t launch_prep_h(const Layout& L, char* ws, const void* H, bool want_hrp, hipStream_t st) {
  const int64_t nblk = L.R_pad / 32;
  const size_t sm = (size_t)32 * L.D * L.esz;
  if (L.dtype == 1) {
    hipLaunchKernelGGL(k_prep_h<__bf16>, dim3((unsigned)nblk), dim3(256), sm, st, (const __bf16*)H,
                       (const int32_t*)(ws + L.off_row_of), (const float*)(ws + L.off_wc), L.D,
                       (__bf16*)(ws + L.off_Hc),
                       want_hrp ? (__bf16*)(ws + L.off_Hrp) : nullptr, (double*)(ws + L.off_sumH_part));
  } else {
    hipLaunchKernelGGL(k_prep_h<float>, dim3((unsigned)nblk), dim3(256), sm, st, (const float*)H,
                       (const int32_t*)(ws + L.off_row_of), (const float*)(ws + L.off_wc), L.D,
                       (float*)(ws + L.off_Hc),
                       want_hrp ? (float*)(ws + L.off_Hrp) : nullptr, (double*)(ws + L.off_sumH_part));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sum_parts, dim3((L.D + 31) / 32), dim3(1024), 0, st,
                     (const double*)(ws + L.off_sumH_part), nblk, L.D, (double*)(ws + L.off_sumH));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------------
// E preparation: block = kEBlkItems items, processed 32 at a time through LDS. Writes the slot-packed Evp
// (when requested) and float64 column sums per block.
// ---------------------------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) k_prep_e(const T* __restrict__ E, int64_t V, int D,
                                                T* __restrict__ Evp, double* __restrict__ sum_part) {
  extern __shared__ char smem_raw[];
  T* tile = (T*)smem_raw;  // [32][D]
  const int tid = threadIdx.x;
  const int upr = D * (int)sizeof(T) / 16;
  double acc0 = 0.0, acc1 = 0.0;  // column sums for d = tid and d = tid + 256
  const int64_t v_begin = (int64_t)blockIdx.x * kEBlkItems;
  for (int ch = 0; ch < kEBlkItems / 32; ++ch) {
    const int64_t v0 = v_begin + ch * 32;
    for (int u = tid; u < 32 * upr; u += 256) {
      const int rr = u / upr, c = u % upr;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (v0 + rr < V) x = *(const u32x4*)((const char*)E + ((v0 + rr) * D) * sizeof(T) + c * 16);
      *(u32x4*)((char*)tile + ((int64_t)rr * D) * sizeof(T) + c * 16) = x;
    }
    __syncthreads();
    if (Evp) {
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
    if (tid < D)
      for (int rr = 0; rr < 32; ++rr) acc0 += (double)(float)tile[rr * D + tid];
    if (tid + 256 < D)
      for (int rr = 0; rr < 32; ++rr) acc1 += (double)(float)tile[rr * D + tid + 256];
    __syncthreads();
  }
  if (tid < D) sum_part[blockIdx.x * (int64_t)D + tid] = acc0;
  if (tid + 256 < D) sum_part[blockIdx.x * (int64_t)D + tid + 256] = acc1;
}

hipError_t launch_prep_e(const Layout& L, char* ws, const void* E, bool want_evp, hipStream_t st) {
  const size_t sm = (size_t)32 * L.D * L.esz;
  if (L.dtype == 1) {
    hipLaunchKernelGGL(k_prep_e<__bf16>, dim3((unsigned)L.n_eblk), dim3(256), sm, st, (const __bf16*)E, L.V,
                       L.D, want_evp ? (__bf16*)(ws + L.off_Evp) : nullptr, (double*)(ws + L.off_sumE_part));
  } else {
    hipLaunchKernelGGL(k_prep_e<float>, dim3((unsigned)L.n_eblk), dim3(256), sm, st, (const float*)E, L.V, L.D,
                       want_evp ? (float*)(ws + L.off_Evp) : nullptr, (double*)(ws + L.off_sumE_part));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sum_parts, dim3((L.D + 31) / 32), dim3(1024), 0, st,
                     (const double*)(ws + L.off_sumE_part), L.n_eblk, L.D, (double*)(ws + L.off_sumE));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------------
// Multi-block exclusive scan of int32 counts, in place: x[i] <- sum_{j<i} x[j] for i <= n (x[n] = total).
// ---------------------------------------------------------------------------------------------------------
constexpr int kScanPerThread = kScanBlock / 1024;

__global__ void __launch_bounds__(1024) k_scan_sums(const int32_t* __restrict__ x, int64_t n,
                                                    int32_t* __restrict__ bsum) {
  __shared__ int sh[16];
  const int64_t b0 = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * kScanPerThread;
  int s = 0;
#pragma unroll
  for (int j = 0; j < kScanPerThread; ++j)
    if (b0 + j < n) s += x[b0 + j];
  int tot;
  block_excl_scan(s, sh, tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

__global__ void __launch_bounds__(1024) k_scan_bsums(int32_t* bsum, int64_t nb) {
  __shared__ int sh[16];
  __shared__ int base;
  if (threadIdx.x == 0) base = 0;
  __syncthreads();
  for (int64_t c0 = 0; c0 < nb; c0 += 1024) {
    const int64_t i = c0 + threadIdx.x;
    const int v = i < nb ? bsum[i] : 0;
    int tot;
    const int ex = block_excl_scan(v, sh, tot);
    if (i < nb) bsum[i] = base + ex;
    __syncthreads();
    if (threadIdx.x == 0) base += tot;
    __syncthreads();
  }
}

__global__ void __launch_bounds__(1024) k_scan_apply(int32_t* __restrict__ x, int64_t n,
                                                     const int32_t* __restrict__ bsum) {
  __shared__ int sh[16];
  const int64_t b0 = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * kScanPerThread;
  int v[kScanPerThread];
  int s = 0;
#pragma unroll
  for (int j = 0; j < kScanPerThread; ++j) {
    v[j] = (b0 + j < n) ? x[b0 + j] : 0;
    s += v[j];
  }
  int tot;
  int run = block_excl_scan(s, sh, tot) + bsum[blockIdx.x];
#pragma unroll
  for (int j = 0; j < kScanPerThread; ++j) {
    if (b0 + j <= n) x[b0 + j] = run;  // entry n receives the grand total
    run += v[j];
  }
}

static hipError_t scan_exclusive(int32_t* x, int64_t n, int32_t* tmp, hipStream_t st) {
  // n + 1 entries are written; blocks cover [0, n] inclusive
  const int64_t nb = (n + 1 + kScanBlock - 1) / kScanBlock;
  hipLaunchKernelGGL(k_scan_sums, dim3((unsigned)nb), dim3(1024), 0, st, x, n, tmp);
  hipLaunchKernelGGL(k_scan_bsums, dim3(1), dim3(1024), 0, st, tmp, nb);
  hipLaunchKernelGGL(k_scan_apply, dim3((unsigned)nb), dim3(1024), 0, st, x, n, tmp);
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
template <bool kScatter>
__global__ void __launch_bounds__(256) k_bucket(const Ctl* __restrict__ ctl, const int2* __restrict__ rptr,
                                                const int32_t* __restrict__ ids, int64_t V, bool rows_side,
                                                int tile, int64_t nsteps_minor, int32_t* __restrict__ cnt,
                                                int2* __restrict__ pairs, int* bad) {
  const int64_t k = (int64_t)blockIdx.x * (blockDim.x / 8) + threadIdx.x / 8;
  const int sub = threadIdx.x % 8;
  if (k >= ctl->n_valid) return;
  const int2 rp = rptr[k];
  int nbad = 0;
  for (int p = rp.x + sub; p < rp.y; p += 8) {
    const int v = ids[p];
    if (v < 0 || v >= V) {
      ++nbad;
      continue;
    }
    const int64_t b = rows_side ? (k / tile) * nsteps_minor + v / 32 : (v / tile) * nsteps_minor + k / 32;
    if (kScatter) {
      const int pos = atomicAdd(&cnt[b], 1);
      pairs[pos] = make_int2((int)k, v);
    } else {
      atomicAdd(&cnt[b], 1);
    }
  }
  if (!kScatter && nbad) atomicAdd(bad, nbad);
}

template <bool kScatter>
__global__ void __launch_bounds__(256) k_bucket_runs(const Ctl* __restrict__ ctl, const int2* __restrict__ rptr,
                                                     const int32_t* __restrict__ ids, int64_t V, bool rows_side,
                                                     int tile, int64_t nsteps_minor, int32_t* __restrict__ cnt,
                                                     int2* __restrict__ pairs, int* bad) {
  const int64_t k = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;  // one row per wave
  const int lane = lane_id();
  if (k >= ctl->n_valid) return;  // the whole wave
  const int2 rp = rptr[k];
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
                       ctl, (const int2*)(ws + L.off_rptr), item_ids, L.V, rows_side, tile, minor, bptr,
                       (int2*)nullptr, &ctl->bad_ids);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = scan_exclusive(bptr, nb, (int32_t*)(ws + L.off_scan), st)) != hipSuccess) return e;
  if (L.nnz > 0) {
    int64_t cblocks = (nb + 255) / 256;
    if (cblocks > 65536) cblocks = 65536;
    hipLaunchKernelGGL(k_copy_i32, dim3((unsigned)cblocks), dim3(256), 0, st, bfill, (const int32_t*)bptr, nb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(runs ? k_bucket_runs<true> : k_bucket<true>, dim3((unsigned)blocks), dim3(256), 0, st,
                       ctl, (const int2*)(ws + L.off_rptr), item_ids, L.V, rows_side, tile, minor, bfill, pairs,
                       (int*)nullptr);
  }
  return hipGetLastError();
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
