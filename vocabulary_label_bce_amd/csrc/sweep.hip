// The two logit-tile sweeps of CutBCE on gfx950 ("Cut Binary Cross Entropy", Section III-A vocabulary
// chunking, Section III-B/III-C rematerialised backward): logits are formed 32x32 at a time in MFMA
// accumulators, turned into loss terms and logit gradients in registers, and fed straight into the gradient
// GEMM. Neither Z nor dZ ever leaves the register file.
//
// Forward sweep (k_rows): a workgroup owns a tile of valid rows (32 per wave) and sweeps one vocabulary split.
//   Z^T = E_step . H_tile^T  (bf16/f32 MFMA, K = D)      -> softplus terms summed per row
//   G   = sigma(Z) - 1/2 - Y (bf16 or f32)               -> dH_tile += G . E_step   (K = 32 items)
// Backward sweep (k_items): a workgroup owns a tile of items (32 per wave) and sweeps every valid row.
//   Z   = H_step . E_tile^T                               -> G = sigma(Z) - 1/2 - Y
//   dE_tile += G^T . H_step                               (K = 32 rows)
// The constant 1/2 taken out of sigma is added back as a rank-1 term (1/2 sum_v E[v] for dH, 1/2 sum_r H[r]
// for dE) in float64 by the finishing kernels: centring keeps the bf16 rounding of G relative to sigma - 1/2,
// which is what carries the gradient signal when logits are small.
#include "common.h"

namespace cutbce {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

template <typename T> __device__ inline typename Elem<T>::Op load_op(const T* p);
template <> __device__ inline bf16x8 load_op<__bf16>(const __bf16* p) { return *(const bf16x8*)p; }
template <> __device__ inline float load_op<float>(const float* p) { return *p; }

// XOR swizzle of 16-byte chunks inside an LDS row of the d-packed operand: lanes reading the same logical
// chunk of 32 consecutive rows hit distinct banks.
template <int CPR> __device__ __host__ constexpr inline int swz(int row) {
  return CPR >= 16 ? (row & 15) : ((row / (16 / CPR)) % CPR);
}

// Pack the 16 accumulator-tile values of a lane into the MFMA operands of the second GEMM.
template <typename T> struct GPack;
template <> struct GPack<__bf16> {
  bf16x8 g[2];
  __device__ inline void set(const float* c) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) g[q][j] = (__bf16)c[q * 8 + j];
  }
  __device__ inline bf16x8 op(int q) const { return g[q]; }
};
template <> struct GPack<float> {
  float g[16];
  __device__ inline void set(const float* c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) g[i] = c[i];
  }
  __device__ inline float op(int q) const { return g[q]; }
};

// Per-lane positive mask for the current 32x32 tile: bit i set iff accumulator register i of this lane is a
// (row, item) positive. Pairs come from the bucket of the current (tile, step); `own` is the first owner
// index of this wave, `stream0` the first streamed index of the step. `owner_is_row` selects which pair
// coordinate the wave owns (rows in the forward sweep, items in the backward sweep).
__device__ inline uint32_t positive_mask(const int2* __restrict__ pairs, int pb, int pe, int own, int stream0,
                                         bool owner_is_row, uint32_t* lmask, int lane) {
  lmask[lane] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  for (int q0 = pb; q0 < pe; q0 += 64) {
    const int q = q0 + lane;
    if (q < pe) {
      const int2 kv = pairs[q];
      const int o = (owner_is_row ? kv.x : kv.y) - own;
      const int sidx = (owner_is_row ? kv.y : kv.x) - stream0;
      if (o >= 0 && o < 32 && sidx >= 0 && sidx < 32) {
        const int tgt = o + 32 * ((sidx >> 2) & 1);
        const int bit = (sidx >> 3) * 4 + (sidx & 3);
        atomicOr(&lmask[tgt], 1u << bit);
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  return lmask[lane];
}

// Choose the number of vocabulary splits S for T row tiles on P persistent workgroups (P a multiple of 8):
// the unit list (s-major) is cut into 8 contiguous per-XCD ranges; efficiency = U / (P * rounds).
__device__ inline int choose_splits(int T, int n_stages, int P, int max_units) {
  int best_s = 1;
  float best = -1.f;
  int smax = n_stages < kMaxSplits ? n_stages : kMaxSplits;
  int cap = max_units / T;
  if (cap < 1) cap = 1;
  if (smax > cap) smax = cap;
  for (int S = 1; S <= smax; ++S) {
    const int U = T * S;
    const int per = (U + 7) / 8;
    const int rounds = (per + P / 8 - 1) / (P / 8);
    const float eff = (float)U / (float)(P * rounds);
    if (eff > best + 1e-6f) {
      best = eff;
      best_s = S;
    }
    if (eff >= 0.95f) break;
  }
  return best_s;
}

constexpr int kMaxUnits = 1024;

template <typename T, int D>
struct StageGeom {
  static constexpr int kEsz = sizeof(T);
  static constexpr int kSI = (D * kEsz <= 256) ? 64 : 32;  // streamed rows/items per stage
  static constexpr int kCPR = D * kEsz / 16;                // 16-byte chunks per d-packed row
  static constexpr int kPartBytes = kSI * D * kEsz;         // bytes of one stage part
  static constexpr int kStageBytes = 2 * kPartBytes;        // d-packed part + slot-packed part
};

// Load one stage (kSI streamed rows of a d-packed matrix X [n][D] and the matching slot-packed blocks of Xsp)
// into registers: `units` 16-byte pieces per thread. Rows >= n_valid_src read as zero.
template <typename T, int D, int NT, bool SP>
struct Stager {
  using G = StageGeom<T, D>;
  static constexpr int kUnitsPart = G::kPartBytes / 16;
  static constexpr int kPer = (kUnitsPart + NT - 1) / NT;
  static constexpr int kSteps = G::kSI / 32;
  u32x4 a[kPer], b[kPer];
  int bp[kSteps + 1];  // bucket pointers of the stage's steps (bucket range of step j: [bp[j], bp[j+1]))
  __device__ inline void load_buckets(const int32_t* __restrict__ bptr, int64_t b0) {
#pragma unroll
    for (int j = 0; j <= kSteps; ++j) bp[j] = bptr[b0 + j];
  }
  __device__ inline void load(const T* __restrict__ X, const T* __restrict__ Xsp, int64_t row0, int64_t n_src,
                              int tid) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int u = tid + q * NT;
      if (u < kUnitsPart) {
        const int r = u / G::kCPR, c = u % G::kCPR;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row0 + r < n_src) x = *(const u32x4*)((const char*)X + (row0 + r) * (int64_t)(D * G::kEsz) + c * 16);
        a[q] = x;
        if (SP) b[q] = *(const u32x4*)((const char*)Xsp + row0 * (int64_t)(D * G::kEsz) + (int64_t)u * 16);
      }
    }
  }
  __device__ inline void store(char* lds, int tid) const {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int u = tid + q * NT;
      if (u < kUnitsPart) {
        const int r = u / G::kCPR, c = u % G::kCPR;
        *(u32x4*)(lds + r * (D * G::kEsz) + ((c ^ swz<G::kCPR>(r)) * 16)) = a[q];
        if (SP) *(u32x4*)(lds + G::kPartBytes + u * 16) = b[q];
      }
    }
  }
};

// A operand of the first GEMM from the d-packed LDS part: streamed row `r` (0..kSI-1), k-step ks.
template <typename T, int D>
__device__ inline typename Elem<T>::Op lds_a(const char* lds, int r, int ks, int lane) {
  using G = StageGeom<T, D>;
  const int k = ks * Elem<T>::kK + (lane / 32) * Elem<T>::kEPL;  // first feature of this lane
  const int byte = k * G::kEsz;
  const int c = byte / 16, w = byte % 16;
  return load_op<T>((const T*)(lds + r * (D * G::kEsz) + ((c ^ swz<G::kCPR>(r)) * 16) + w));
}

// B operand of the second GEMM from the slot-packed LDS part: 32-block `blk` of the stage, d-block db, group g.
template <typename T, int D>
__device__ inline typename Elem<T>::Op lds_b(const char* lds, int blk, int db, int g, int lane) {
  using G = StageGeom<T, D>;
  const T* p = (const T*)(lds + G::kPartBytes) + (int64_t)blk * 32 * D + slot_off<T>(D, db, g, lane);
  return load_op<T>(p);
}

struct RowsArgs {
  const void* Hc;
  const void* E;
  const void* Evp;
  Ctl* ctl;
  const int32_t* bptr;
  const int2* pairs;
  int64_t V, V_pad, n_vs, R_pad;
  float* dhpart;   // [units][RW][D]
  float2* rowpart; // [units][RW]
};

// ---------------------------------------------------------------------------------------------------------
// Forward sweep. Persistent: gridDim.x workgroups (a multiple of 8, one per CU); units (split s, row tile t)
// are assigned in contiguous per-XCD ranges so that the workgroups sharing an L2 stream the same part of E.
// ---------------------------------------------------------------------------------------------------------
template <typename T, int D, int NW, bool WITH_DH>
__global__ void __launch_bounds__(NW * 64) k_rows(RowsArgs a) {
  using EL = Elem<T>;
  using G = StageGeom<T, D>;
  constexpr int NT = NW * 64, RW = NW * 32, KS = D / EL::kK, NDB = D / 32;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  uint32_t* lmask_all = (uint32_t*)(lds + 2 * G::kStageBytes);
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
  uint32_t* lmask = lmask_all + wave * 64;
  const T* __restrict__ Hc = (const T*)a.Hc;
  const T* __restrict__ E = (const T*)a.E;
  const T* __restrict__ Evp = (const T*)a.Evp;

  const int n_valid = a.ctl->n_valid;
  const int Tt = (n_valid + RW - 1) / RW;
  if (Tt == 0) return;
  const int n_stages = (int)(a.V_pad / G::kSI);
  const int P = gridDim.x;
  const int S = choose_splits(Tt, n_stages, P, kMaxUnits);
  if (blockIdx.x == 0 && tid == 0) a.ctl->splits = S;
  const int U = Tt * S;
  const int x = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int start = (int)(((int64_t)x * U) / 8), cnt = (int)(((int64_t)(x + 1) * U) / 8) - start;

  for (int idx = slot; idx < cnt; idx += P / 8) {
    const int u = start + idx;
    const int s = u / Tt, t = u % Tt;
    const int st0 = (int)(((int64_t)s * n_stages) / S), st1 = (int)(((int64_t)(s + 1) * n_stages) / S);
    const int r_base = t * RW + wave * 32;

    typename EL::Op hop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      hop[ks] = load_op<T>(Hc + (int64_t)(r_base + lane % 32) * D + ks * EL::kK + (lane / 32) * EL::kEPL);
    f32x16 acc[WITH_DH ? NDB : 1];
    if (WITH_DH)
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    float e_acc = 0.f, posz = 0.f;

    Stager<T, D, NT, WITH_DH> pf;
    constexpr int NSS = G::kSI / 32;
    const int64_t bbase = (int64_t)t * a.n_vs;
    __syncthreads();  // previous unit finished reading LDS
    pf.load(E, Evp, (int64_t)st0 * G::kSI, a.V, tid);
    pf.load_buckets(a.bptr, bbase + (int64_t)st0 * NSS);
    pf.store(lds, tid);
    __syncthreads();

    for (int st = st0; st < st1; ++st) {
      const char* buf = lds + ((st - st0) & 1) * G::kStageBytes;
      const bool more = st + 1 < st1;
      int bcur[NSS + 1];
#pragma unroll
      for (int j = 0; j <= NSS; ++j) bcur[j] = __builtin_amdgcn_readfirstlane(pf.bp[j]);
      if (more) {
        pf.load(E, Evp, (int64_t)(st + 1) * G::kSI, a.V, tid);
        pf.load_buckets(a.bptr, bbase + (int64_t)(st + 1) * NSS);
      }
#pragma unroll
      for (int ss = 0; ss < NSS; ++ss) {
        const int v0 = st * G::kSI + ss * 32;
        typename EL::Op aop[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) aop[ks] = lds_a<T, D>(buf, ss * 32 + lane % 32, ks, lane);
        f32x16 z = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) z = EL::mma(aop[ks], hop[ks], z);

        const int pb = bcur[ss], pe = bcur[ss + 1];
        uint32_t pm = 0u;
        if (pe > pb) pm = positive_mask(a.pairs, pb, pe, r_base, v0, true, lmask, lane);

        float c[16];
        float s1 = 0.f, prod = 1.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float zi = z[i];
          const float az = __builtin_fabsf(zi);
          const float tt = __builtin_amdgcn_exp2f(az * -kLog2e);
          const float w1 = 1.f + tt;
          prod *= w1;
          s1 += az;
          if (WITH_DH) c[i] = __builtin_copysignf(__builtin_amdgcn_rcpf(w1) - 0.5f, zi);
        }
        e_acc += 0.5f * s1 + kLn2 * (__builtin_amdgcn_logf(prod) - 16.f);
        if (pm) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (pm & (1u << i)) {
              posz += z[i];
              if (WITH_DH) c[i] -= 1.f;
            }
        }
        if (WITH_DH) {
          GPack<T> gp;
          gp.set(c);
          typename EL::Op bop[NDB][EL::kGroups];
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < EL::kGroups; ++g) bop[db][g] = lds_b<T, D>(buf, ss, db, g, lane);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < EL::kGroups; ++g) acc[db] = EL::mma(gp.op(g), bop[db][g], acc[db]);
        }
      }
      if (more) pf.store(lds + ((st + 1 - st0) & 1) * G::kStageBytes, tid);
      __syncthreads();
    }

    // unit results: per-row loss parts and the dH partial of this split
    const int64_t urow = (int64_t)u * RW + wave * 32;  // row of the unit-major partial buffers
    const float e_tot = e_acc + __shfl_xor(e_acc, 32, 64);
    const float p_tot = posz + __shfl_xor(posz, 32, 64);
    if (lane < 32) a.rowpart[urow + lane] = make_float2(e_tot, p_tot);
    if (WITH_DH) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          a.dhpart[(urow + acc_pos(i, lane / 32)) * D + db * 32 + lane % 32] = acc[db][i];
    }
  }
}

struct ItemsArgs {
  const void* Hc;
  const void* Hrp;
  const void* E;
  const Ctl* ctl;
  const int32_t* bptr;
  const int2* pairs;
  const double* sumH;
  const float* grad_loss;
  void* dE;
  int64_t V, n_rs;
};

// ---------------------------------------------------------------------------------------------------------
// Backward dE sweep: workgroup = item tile (32 items per wave), sweeping all valid rows.
// ---------------------------------------------------------------------------------------------------------
template <typename T, int D, int NW>
__global__ void __launch_bounds__(NW * 64) k_items(ItemsArgs a) {
  using EL = Elem<T>;
  using G = StageGeom<T, D>;
  constexpr int NT = NW * 64, IW = NW * 32, KS = D / EL::kK, NDB = D / 32;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  uint32_t* lmask = (uint32_t*)(lds + 2 * G::kStageBytes) + (threadIdx.x / 64) * 64;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
  const T* __restrict__ Hc = (const T*)a.Hc;
  const T* __restrict__ Hrp = (const T*)a.Hrp;
  const T* __restrict__ E = (const T*)a.E;

  const int t = blockIdx.x;
  const int64_t v_own0 = (int64_t)t * IW + wave * 32;  // first item of this wave
  const int64_t v_mine = v_own0 + lane % 32;
  typename EL::Op eop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (v_mine < a.V) {
      eop[ks] = load_op<T>(E + v_mine * D + ks * EL::kK + (lane / 32) * EL::kEPL);
    } else {
      eop[ks] = typename EL::Op{};
    }
  }
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  const int n_valid = a.ctl->n_valid;
  const int n_st = (n_valid + G::kSI - 1) / G::kSI;
  Stager<T, D, NT, true> pf;
  constexpr int NSS = G::kSI / 32;
  const int64_t bbase = (int64_t)t * a.n_rs;
  if (n_st > 0) {
    pf.load(Hc, Hrp, 0, (int64_t)n_valid, tid);
    pf.load_buckets(a.bptr, bbase);
    pf.store(lds, tid);
  }
  __syncthreads();
  for (int st = 0; st < n_st; ++st) {
    const char* buf = lds + (st & 1) * G::kStageBytes;
    const bool more = st + 1 < n_st;
    int bcur[NSS + 1];
#pragma unroll
    for (int j = 0; j <= NSS; ++j) bcur[j] = __builtin_amdgcn_readfirstlane(pf.bp[j]);
    if (more) {
      pf.load(Hc, Hrp, (int64_t)(st + 1) * G::kSI, (int64_t)n_valid, tid);
      pf.load_buckets(a.bptr, bbase + (int64_t)(st + 1) * NSS);
    }
#pragma unroll
    for (int ss = 0; ss < NSS; ++ss) {
      const int r0 = st * G::kSI + ss * 32;
      typename EL::Op aop[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) aop[ks] = lds_a<T, D>(buf, ss * 32 + lane % 32, ks, lane);
      f32x16 z = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) z = EL::mma(aop[ks], eop[ks], z);

      const int pb = bcur[ss], pe = bcur[ss + 1];
      uint32_t pm = 0u;
      if (pe > pb) pm = positive_mask(a.pairs, pb, pe, (int)v_own0, r0, false, lmask, lane);

      float c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float tt = __builtin_amdgcn_exp2f(z[i] * -kLog2e);
        c[i] = __builtin_amdgcn_rcpf(1.f + tt) - 0.5f;
      }
      if (pm) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (pm & (1u << i)) c[i] -= 1.f;
      }
      GPack<T> gp;
      gp.set(c);
      typename EL::Op bop[NDB][EL::kGroups];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < EL::kGroups; ++g) bop[db][g] = lds_b<T, D>(buf, ss, db, g, lane);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < EL::kGroups; ++g) acc[db] = EL::mma(gp.op(g), bop[db][g], acc[db]);
    }
    if (more) pf.store(lds + ((st + 1) & 1) * G::kStageBytes, tid);
    __syncthreads();
  }

  // dE[v][d] = s * g * (acc + 1/2 sum_r H[r][d])
  const double sc = a.ctl->scale * (double)a.grad_loss[0];
  const float scf = (float)sc;
  T* __restrict__ dE = (T*)a.dE;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d = db * 32 + lane % 32;
    const float half = (float)(0.5 * a.sumH[d]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t v = v_own0 + acc_pos(i, lane / 32);
      if (v < a.V) dE[v * D + d] = (T)(scf * (acc[db][i] + half));
    }
  }
}

// ---------------------------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------------------------
static int g_cus = 0;
static int cu_count() {
  if (g_cus == 0) {
    int dev = 0;
    hipGetDevice(&dev);
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cus = n;
  }
  return g_cus;
}

template <typename T, int D, int NW, bool WITH_DH>
static hipError_t rows_launch(const Layout& L, char* ws, const void* E, hipStream_t st) {
  using G = StageGeom<T, D>;
  RowsArgs a;
  a.Hc = ws + L.off_Hc;
  a.E = E;
  a.Evp = ws + L.off_Evp;
  a.ctl = (Ctl*)(ws + L.off_ctl);
  a.bptr = (const int32_t*)(ws + L.off_bptr_r);
  a.pairs = (const int2*)(ws + L.off_pairs_r);
  a.V = L.V;
  a.V_pad = L.V_pad;
  a.n_vs = L.n_vs;
  a.R_pad = L.R_pad;
  a.dhpart = (float*)(ws + L.off_dhpart);
  a.rowpart = (float2*)(ws + L.off_rowpart);
  const size_t sm = 2 * G::kStageBytes + NW * 64 * 4;
  auto kern = k_rows<T, D, NW, WITH_DH>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  const int P = (cu_count() / 8) * 8;
  hipLaunchKernelGGL(kern, dim3(P > 0 ? P : 8), dim3(NW * 64), sm, st, a);
  return hipGetLastError();
}

template <typename T, int D, int NW>
static hipError_t items_launch(const Layout& L, char* ws, const void* E, const float* grad_loss, void* dE,
                               hipStream_t st) {
  using G = StageGeom<T, D>;
  ItemsArgs a;
  a.Hc = ws + L.off_Hc;
  a.Hrp = ws + L.off_Hrp;
  a.E = E;
  a.ctl = (const Ctl*)(ws + L.off_ctl);
  a.bptr = (const int32_t*)(ws + L.off_bptr_i);
  a.pairs = (const int2*)(ws + L.off_pairs_i);
  a.sumH = (const double*)(ws + L.off_sumH);
  a.grad_loss = grad_loss;
  a.dE = dE;
  a.V = L.V;
  a.n_rs = L.n_rs;
  const size_t sm = 2 * G::kStageBytes + NW * 64 * 4;
  auto kern = k_items<T, D, NW>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)L.n_vt), dim3(NW * 64), sm, st, a);
  return hipGetLastError();
}

#define CUTBCE_DISPATCH(DT, FN, ...)                                                             \
  do {                                                                                           \
    if ((DT) == 1) {                                                                             \
      switch (L.D) {                                                                             \
        case 64: return FN<__bf16, 64, sweep_waves(1, 64)>(__VA_ARGS__);                        \
        case 128: return FN<__bf16, 128, sweep_waves(1, 128)>(__VA_ARGS__);                     \
        case 256: return FN<__bf16, 256, sweep_waves(1, 256)>(__VA_ARGS__);                     \
        case 512: return FN<__bf16, 512, sweep_waves(1, 512)>(__VA_ARGS__);                     \
      }                                                                                          \
    } else {                                                                                     \
      switch (L.D) {                                                                             \
        case 64: return FN<float, 64, sweep_waves(0, 64)>(__VA_ARGS__);                         \
        case 128: return FN<float, 128, sweep_waves(0, 128)>(__VA_ARGS__);                      \
        case 256: return FN<float, 256, sweep_waves(0, 256)>(__VA_ARGS__);                      \
      }                                                                                          \
    }                                                                                            \
    return hipErrorInvalidValue;                                                                 \
  } while (0)

template <typename T, int D, int NW>
static hipError_t rows_any(const Layout& L, char* ws, const void* E, bool with_dh, hipStream_t st) {
  return with_dh ? rows_launch<T, D, NW, true>(L, ws, E, st) : rows_launch<T, D, NW, false>(L, ws, E, st);
}

hipError_t launch_rows_sweep(const Layout& L, char* ws, const void* E, bool with_dh, hipStream_t st) {
  CUTBCE_DISPATCH(L.dtype, rows_any, L, ws, E, with_dh, st);
}

hipError_t launch_items_sweep(const Layout& L, char* ws, const void* E, const float* grad_loss, void* dE,
                              hipStream_t st) {
  CUTBCE_DISPATCH(L.dtype, items_launch, L, ws, E, grad_loss, dE, st);
}

}  // namespace cutbce
