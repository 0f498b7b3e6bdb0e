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
//
// Both sweeps share one software-pipelined step engine. Iteration i of a wave issues the MFMAs of the logit
// tile of step i and of the gradient GEMM of step i-1, then reads the operands of step i+1 and evaluates the
// epilogue of step i on the vector ALU; none depends on another, so while one wave runs its MFMAs the other
// wave of the SIMD can run its vector work. Streamed operands reach LDS by direct buffer loads (global -> LDS,
// no registers) into two rings, one for the d-packed operand of the logit GEMM and one for the slot-packed
// operand of the gradient GEMM; workgroup barriers come every few steps (see Geo).
//
// The forward sweep also serves full-vocabulary scoring (top-k per row, Section III-E's evaluation) with a
// running top list per lane in place of the loss epilogue, and can count the Cut Metrics of Section III-D.
#include <atomic>
#include <type_traits>

#include "common.h"

namespace cutbce {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0)); }

template <typename T> __device__ inline typename Elem<T>::Op load_op(const T* p);
template <> __device__ inline bf16x8 load_op<__bf16>(const __bf16* p) { return *(const bf16x8*)p; }
template <> __device__ inline float load_op<float>(const float* p) { return *p; }

typedef __attribute__((address_space(3))) void lds_void;

// XOR swizzle of 16-byte chunks inside an LDS row of the d-packed operand: lanes reading the same logical
// chunk of 32 consecutive rows hit distinct banks.
template <int CPR> __device__ __host__ constexpr inline int swz(int row) {
  constexpr int rows_per_group = CPR >= 16 ? 1 : 16 / CPR;
  return CPR >= 16 ? (row & 15) : ((row / rows_per_group) % CPR);
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
// f16 G tile of the bf16 dE sweep (its B operand, the weighted rows, is f16 scaled by a power of two): three more
// bits than bf16 for c = sigma(z) - 1/2 - y, which matters at positives, where c lies in [-3/2, -1/2].
struct GPackF16 {
  f16x8 g[2];
  __device__ inline void set(const float* c) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) g[q][j] = (_Float16)c[q * 8 + j];
  }
  __device__ inline f16x8 op(int q) const { return g[q]; }
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
constexpr int kMaxUnits = 1024;
__device__ inline int choose_splits(int T, int n_steps, int P) {
  int best_s = 1;
  float best = -1.f;
  int smax = n_steps / 8 < kMaxSplits ? n_steps / 8 : kMaxSplits;  // at least 8 steps per unit
  if (smax < 1) smax = 1;
  int cap = kMaxUnits / T;
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

// ---------------------------------------------------------------------------------------------------------
// Per-lane running top-KT list for full-vocabulary scoring: values in descending order, ids alongside. Items
// reach a lane in increasing id order, so a strict comparison keeps the smaller id first among equal logits;
// merging lists from other lanes or splits applies the full rule (larger logit, then smaller id).
// ---------------------------------------------------------------------------------------------------------
template <int KT>
struct TopK {
  float v[KT];
  int id[KT];
  __device__ inline void init() {
#pragma unroll
    for (int q = 0; q < KT; ++q) {
      v[q] = -__builtin_inff();
      id[q] = -1;
    }
  }
  // insert (x, i) when it ranks before the last entry; `later` = every listed id is smaller than i
  template <bool LATER>
  __device__ inline void insert(float x, int i) {
#pragma unroll
    for (int q = 0; q < KT; ++q) {
      const bool sw = LATER ? x > v[q] : (x > v[q] || (x == v[q] && (unsigned)i < (unsigned)id[q]));
      const float tv = v[q];
      const int ti = id[q];
      v[q] = sw ? x : tv;
      id[q] = sw ? i : ti;
      x = sw ? tv : x;
      i = sw ? ti : i;
    }
  }
  __device__ inline float last() const { return v[KT - 1]; }
};

// ---------------------------------------------------------------------------------------------------------
// Geometry of the step engine for (T, D, NW waves, GRAD = gradient GEMM present).
//
// The streamed operand moves through two LDS rings, one 32-row block per step: the d-packed block of step j
// (A, read for the logit GEMM during iteration j - 1) and its slot-packed copy (B, read by the gradient GEMM
// during iteration j + 1). Workgroup barriers come every kK iterations (at iterations that are multiples of
// kK): a barrier costs a wait of every wave for the slowest, and kK = 2 at 8 KB steps measured best. With
// kS = 1 a barrier waits for all loads but those issued in the iteration just before it. Then:
//   A(j) is loaded at iteration j - kLA into slot j % kNA; B(j) at iteration j - kLB into slot j % kNB, with
//   kLA >= kK + 1 + kS, kLB >= kK - 1 + kS     (a barrier separates landing from reading),
//   kNA >= kLA + kK - 1, kNB >= kLB + kK + 1     (a barrier separates the last read of a slot from its
//                                                 refill).
// ---------------------------------------------------------------------------------------------------------
#ifndef CUTBCE_LOAD_SLACK
#define CUTBCE_LOAD_SLACK 1  // iterations whose ring loads a barrier lets stay in flight (steps up to 16 KB)
#endif
#ifndef CUTBCE_STEPS_PER_BARRIER
#define CUTBCE_STEPS_PER_BARRIER 0  // 0: by step size
#endif
template <typename T, int D, int NW, bool GRAD>
struct Geo {
  static constexpr int kEsz = sizeof(T);
  static constexpr int kStepBytes = 32 * D * kEsz;  // one 32-row block of an operand
  static constexpr int kK = CUTBCE_STEPS_PER_BARRIER > 0 ? (kStepBytes <= 8192 ? CUTBCE_STEPS_PER_BARRIER : 1)
                            : (kStepBytes <= 4096 ? 4 : kStepBytes <= 8192 ? 2 : 1);
  static constexpr int kS = kStepBytes <= 16384 ? CUTBCE_LOAD_SLACK : 0;
  static constexpr int kLA = kK + 1 + kS, kLB = kK - 1 + kS;
  static constexpr int kNA = kLA + kK - 1, kNB = GRAD ? kLB + kK + 1 : 0;
  static constexpr int kCPR = D * kEsz / 16;                         // 16-byte chunks per d-packed row
  static constexpr int kLoadB = (kStepBytes / NW >= 1024) ? 16 : 4;  // bytes per lane per DMA load
  static constexpr int kWaveBytes = 64 * kLoadB;                     // bytes one wave instruction moves
  static constexpr int kLoadsPerPart = kStepBytes / kWaveBytes / NW;
  // vector-memory loads an iteration issues (ring blocks; the bucket-pointer loads come once per 64 steps and
  // only make the following barrier wait longer)
  static constexpr int kLoadsPerIter = kLoadsPerPart * (GRAD ? 2 : 1);
  static constexpr int kInFlight = kS * kLoadsPerIter;  // loads a barrier lets stay in flight
  static constexpr int kLdsBytes = (kNA + kNB) * kStepBytes + NW * 256;
  static_assert(kLoadsPerPart >= 1 && kStepBytes % (kWaveBytes * NW) == 0, "load split");
  static_assert(kLoadsPerIter <= 63, "vmcnt range");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

// Ring barrier. vmcnt(N): this wave's DMA loads older than the last N have landed in LDS. lgkmcnt(0): this
// wave's own LDS reads have returned -- the compiler may sink the MFMAs that consume them (and their waits)
// past this asm statement, and a read still queued at the LDS must not see a slot another wave refills
// after the barrier.
template <int N> __device__ inline void wait_vm_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// A operand of the logit GEMM from a d-packed LDS block: streamed row `r` (0..31), k-step ks.
template <typename T, int D>
__device__ inline typename Elem<T>::Op lds_a(const char* blk, int r, int ks, int lane) {
  constexpr int esz = sizeof(T), cpr = D * esz / 16;
  const int k = ks * Elem<T>::kK + (lane / 32) * Elem<T>::kEPL;  // first feature of this lane
  const int byte = k * esz;
  const int c = byte / 16, w = byte % 16;
  return load_op<T>((const T*)(blk + r * (D * esz) + ((c ^ swz<cpr>(r)) * 16) + w));
}

// B operand of the gradient GEMM from a slot-packed LDS block: d-block db, group g.
template <typename T, int D>
__device__ inline typename Elem<T>::Op lds_b(const char* blk, int db, int g, int lane) {
  return load_op<T>((const T*)blk + slot_off<T>(D, db, g, lane));
}

// Epilogue of the forward sweep for one 32x32 tile (16 values per lane). With t = e^-z and w = 1 + t,
//   softplus(z) = ln 2 + z + [ln w - ln 2]   and   sigma(z) = 1/w,
// e_acc gathers the bracket (it is 0 for z = 0, so zero padding adds nothing), 16 logits at a time as
// ln 2 * (log2(prod w) - 16); z and ln 2 are added back per row in float64 (sum_v z_rv = H[r] . sum_v E[v]).
// With GRAD it also forms c = sigma(z) - 1/2 (minus 1 at positives).
// w grows without bound for negative z, so this form holds while the tile's product of w stays below
// kFastProd (then every partial product does too, and the reciprocal of each quad's product is a normal float).
// A tile beyond it takes the |z| form instead, whose factors lie in (1, 2]:
//   softplus(z) - z - ln 2 = [|z|/2 + ln((1 + e^-|z|) / 2)] - z/2,   c = sign(z) (1/(1 + e^-|z|) - 1/2).
constexpr float kFastProd = 0x1p120f;

// c_i = 1/w_i - 1/2 for 4Q factors w_i >= 1 (16 by default) with pair products w2 and quad products w4 (each below 2^126):
// one reciprocal per quad, then down the product tree (batch inversion): 1/(w0 w1) = w2 w3 / (w0 w1 w2 w3),
// 1/w0 = w1 / (w0 w1), ...; each 1/w_i picks up two extra roundings.
template <int Q = 4>
__device__ inline void inv_minus_half(const float* w, const float* w2, const float* w4, float* c) {
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const float r4 = __builtin_amdgcn_rcpf(w4[q]);
    const float ra = r4 * w2[2 * q + 1], rb = r4 * w2[2 * q];
    c[4 * q] = ra * w[4 * q + 1] - 0.5f;
    c[4 * q + 1] = ra * w[4 * q] - 0.5f;
    c[4 * q + 2] = rb * w[4 * q + 3] - 0.5f;
    c[4 * q + 3] = rb * w[4 * q + 2] - 0.5f;
  }
}

template <bool GRAD, bool HASPOS, bool LOSS = true>
__device__ inline void epi_rows(const f32x16& z, uint32_t pm, float* c, float& e_acc, float& posz) {
  // The product is formed over adjacent pairs, then quads, then the whole tile.
  float w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = 1.f + __builtin_amdgcn_exp2f(z[i] * -kLog2e);
  float w2[8], w4[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) w2[i] = w[2 * i] * w[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) w4[i] = w2[2 * i] * w2[2 * i + 1];
  const float wp = (w4[0] * w4[1]) * (w4[2] * w4[3]);
  if (GRAD) inv_minus_half(w, w2, w4, c);
  float e_inc = LOSS ? kLn2 * (__builtin_amdgcn_logf(wp) - 16.f) : 0.f;
  // taken by the whole wave when any lane needs it (a branch around the rarely run code; all lanes may run it)
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(wp <= kFastProd)) != 0, 0)) {
    // u_i = -|z_i| log2(e); wa_i = 1 + 2^u_i in (1, 2], so the product of 16 of them cannot overflow
    float u[16], wa[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      u[i] = __builtin_fabsf(z[i]) * -kLog2e;
      wa[i] = 1.f + __builtin_amdgcn_exp2f(u[i]);
    }
    float a2[8], a4[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) a2[i] = wa[2 * i] * wa[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) a4[i] = a2[2 * i] * a2[2 * i + 1];
    if (GRAD) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float r4 = __builtin_amdgcn_rcpf(a4[q]);
        const float ra = r4 * a2[2 * q + 1], rb = r4 * a2[2 * q];
        const float r[4] = {ra * wa[4 * q + 1], ra * wa[4 * q], rb * wa[4 * q + 3], rb * wa[4 * q + 2]};
#pragma unroll
        for (int k = 0; k < 4; ++k) c[4 * q + k] = __builtin_copysignf(r[k] - 0.5f, z[4 * q + k]);
      }
    }
    if (LOSS) {
      float us = 0.f, zs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        us += u[i];
        zs += z[i];
      }
      const float pa = (a4[0] * a4[1]) * (a4[2] * a4[3]);
      // sum_i [ln(1 + e^-|z_i|) - ln 2 + |z_i| / 2 - z_i / 2]
      e_inc = kLn2 * (__builtin_amdgcn_logf(pa) - 16.f - 0.5f * us) - 0.5f * zs;
    }
  }
  if (LOSS) e_acc += e_inc;
  if (HASPOS) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (pm & (1u << i)) {
        posz += z[i];
        if (GRAD) c[i] -= 1.f;
      }
  }
}

// Epilogue of the backward sweep: c = sigma(z) - 1/2 = 1/(1 + e^-z) - 1/2 (minus 1 at positives); e^-z may
// overflow to +inf, which gives exactly -1/2. (Batch inversion as in the forward measured 6% slower here: the
// product tree lengthens each lane's dependency chain more than the 12 saved reciprocals gain.)
template <bool HASPOS>
__device__ inline void epi_items(const f32x16& z, uint32_t pm, float* c) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float tt = __builtin_amdgcn_exp2f(z[i] * -kLog2e);
    c[i] = __builtin_amdgcn_rcpf(1.f + tt) - 0.5f;
  }
  if (HASPOS) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (pm & (1u << i)) c[i] -= 1.f;
  }
}

// ---------------------------------------------------------------------------------------------------------
// The step engine. Owner operands (H rows in the forward, E items in the backward) sit in registers; the
// streamed matrix X (E or Hc) and its slot-packed copy Xsp flow through the LDS rings.
//   FWD: epilogue = softplus (+ sigma with GRAD), owner = rows; !FWD: epilogue = sigma, owner = items.
// Runs steps [j0, j1) of 32 streamed rows; bucket pointers of step j are bptr[bbase + j], bptr[bbase + j + 1].
// Two schedules, both with the gradient GEMM of step i-1 (on the G tile packed in iteration i-1) in iteration i:
//  - kPrefetch (the A operands of a step fit in 32 registers per lane: bf16 D <= 128, f32 D <= 64; also the
//    bf16 D = 512 scoring sweep, whose one wave per SIMD has 512 registers): iteration i runs the logit GEMM of
//    step i on A operands read from LDS during iteration i-1, reads those of step i+1, and evaluates the
//    epilogue of step i;
//  - otherwise the logit GEMM of step i+1 runs in iteration i with its A operands read next to each MFMA, two
//    logit tiles alternating, and the epilogue of step i uses the tile formed in iteration i-1.
// Ring loads, their slots and the barrier every kK iterations follow Geo; bucket pointers come 64 steps at a
// time (bkt_*), their refill riding on a barrier iteration.
// ---------------------------------------------------------------------------------------------------------
// DB0, NDBE: the gradient GEMM covers the d-blocks [DB0, DB0 + NDBE) of the 32-wide blocks of D (acc holds
// NDBE tiles); LOSS = false skips the loss sums of the forward epilogue (a second pass over the other d-blocks).
template <typename T, int D, int NW, bool FWD, bool GRAD, bool MET = false, int KT = 0, int DB0 = 0,
          int NDBE = D / 32, bool LOSS = true, bool F16G = false>
struct Engine {
  using EL = Elem<T>;
  static_assert(!F16G || (std::is_same<T, __bf16>::value && GRAD), "f16 G tiles: bf16 sweeps with a gradient GEMM");
  using GP = typename std::conditional<F16G, GPackF16, GPack<T>>::type;
  using G = Geo<T, D, NW, GRAD>;
  static constexpr int KS = D / EL::kK, NDB = D / 32;
  using Op = typename EL::Op;
  static constexpr bool kPrefetch = KS * (int)sizeof(Op) <= 128 || (FWD && sizeof(T) == 2 && D == 512);

  char* lds;
  int wave, lane;
  const T* X;
  const T* Xsp;
  int64_t nX;
  const int32_t* bptr;
  const int2* pairs;
  int64_t bbase;
  int own0;  // first owner index of this wave (compact row or item)
  int j0, j1;
  bool apply_pos = true;  // false: positives are only counted (Cut Metrics); the finish adds their terms

  uint32_t lds_s;  // LDS byte address of `lds`, wave-uniform (scalar): DMA destinations are formed in SGPRs

  __device__ inline void setup(char* l, int w, int ln) {
    lds = l;
    wave = __builtin_amdgcn_readfirstlane(w);
    lane = ln;
    lds_s = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_void*)l);
  }
  __device__ inline char* ringA(int rel) const { return lds + (rel % G::kNA) * G::kStepBytes; }
  __device__ inline uint32_t* lmask() const {
    return (uint32_t*)(lds + (G::kNA + G::kNB) * G::kStepBytes) + wave * 64;
  }
  __device__ inline int clampj(int rel) const { return j0 + rel < j1 ? j0 + rel : j1 - 1; }

  // d-packed block of step j0 + rel into A slot `slot` = rel % NA (rows >= nX read as zero).
  __device__ inline void dma_a(int rel) const { dma_a(rel, rel % G::kNA); }
  __device__ inline void dma_a(int rel, int slot) const {
    const int64_t row0 = (int64_t)clampj(rel) * 32;
    const char* xa = (const char*)X + row0 * (int64_t)(D * G::kEsz);
    const int64_t rem = (nX - row0) * (int64_t)(D * G::kEsz);
    const int nrec = rem <= 0 ? 0 : (rem > (int64_t)G::kStepBytes ? G::kStepBytes : (int)rem);
    __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)xa, (short)0, nrec, 0x00020000);
    const uint32_t dst = lds_s + slot * G::kStepBytes;
#pragma unroll
    for (int q = 0; q < G::kLoadsPerPart; ++q) {
      const int inst = wave + q * NW;                           // wave instruction index within the block
      const int pos = inst * G::kWaveBytes + lane * G::kLoadB;  // LDS byte written by this lane
      const int row = pos / (D * G::kEsz);
      const int within = pos % (D * G::kEsz);
      const int lchunk = (within / 16) ^ swz<G::kCPR>(row);
      const int voff = row * (D * G::kEsz) + lchunk * 16 + within % 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(size_t)(dst + inst * G::kWaveBytes), G::kLoadB, voff,
                                               0, 0, 0);
    }
  }
  // slot-packed block of step j0 + rel into B slot `slot` = rel % NB (a contiguous copy).
  __device__ inline void dma_b(int rel) const { dma_b(rel, rel % (G::kNB ? G::kNB : 1)); }
  __device__ inline void dma_b(int rel, int slot) const {
    const int64_t row0 = (int64_t)clampj(rel) * 32;
    const char* xb = (const char*)Xsp + row0 * (int64_t)(D * G::kEsz);
    __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)xb, (short)0, G::kStepBytes, 0x00020000);
    const uint32_t dst = lds_s + (G::kNA + slot) * G::kStepBytes;
#pragma unroll
    for (int q = 0; q < G::kLoadsPerPart; ++q) {
      const int inst = wave + q * NW;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(size_t)(dst + inst * G::kWaveBytes), G::kLoadB,
                                               inst * G::kWaveBytes + lane * G::kLoadB, 0, 0, 0);
    }
  }
  // Bucket pointers, 64 steps at a time: lane l of block b holds those of step 64b + l (bk_lo) and of the step
  // after it (bk_hi); a step reads its pair with two lane reads. The next block is loaded a whole block ahead,
  // so no step waits on a recent load (a load consumed one step after it is issued would make the wave wait
  // for every earlier memory operation, the ring loads included).
  int bk_lo, bk_hi, bn_lo, bn_hi;
  __device__ inline void bkt_load(int b, int& lo, int& hi) const {
    int x = j0 + 64 * b + lane;
    x = x < j1 - 1 ? x : j1 - 1;  // steps past the unit are never used
    lo = bptr[bbase + x];
    hi = bptr[bbase + x + 1];
  }
  __device__ inline void bkt_init() {
    bkt_load(0, bk_lo, bk_hi);
    bkt_load(1, bn_lo, bn_hi);
  }
  // Step j > 0 starts block j / 64 (j % 64 == 0). Steps that are multiples of 64 are barrier iterations (kK
  // divides 64), so this rare refill sits in the barrier's branch and adds none to the other iterations.
  __device__ inline void bkt_next(int j) {
    bk_lo = bn_lo;
    bk_hi = bn_hi;
    bkt_load((j >> 6) + 1, bn_lo, bn_hi);
  }
  __device__ inline void bkt_get(int j, int& pb, int& pe) const {
    pb = __builtin_amdgcn_readlane(bk_lo, j & 63);
    pe = __builtin_amdgcn_readlane(bk_hi, j & 63);
  }
  // Start of iteration j's barrier (taken when j % kK == 0), with the bucket block refill it carries.
  __device__ inline void barrier_at(int j) {
    static_assert(64 % G::kK == 0, "bucket blocks start on barrier iterations");
    wait_vm_and_barrier<G::kInFlight>();
    if ((j & 63) == 0 && j > 0) bkt_next(j);
  }

  // Runs the sweep; `own` holds the owner operand for every k-step. On return acc holds the gradient tile
  // (GRAD) and e_acc / posz the forward row sums (FWD).
  //
  // Prefetching schedule: iteration i does the logit GEMM of step i and the gradient GEMM of step i-1 (with the
  // G tile of step i-1) on the matrix cores, reads the A operands of step i+1, and runs the epilogue of step i
  // (giving G(i)) on the vector ALU. Only the epilogue depends on another of these (the logit GEMM), so the
  // gradient MFMAs interleave with it, and the scalar work of the ring loads fills the gaps of the logit
  // GEMM's dependent MFMA chain. Each wave keeps one logit tile, one G tile and the A operands of its next
  // logit GEMM in registers. A last iteration i = n finishes the pipeline (no loads, no logit GEMM).
  __device__ inline void run(const Op* own, f32x16* acc, float& e_acc, float& posz, int* met,
                             TopK<KT ? KT : 1>* tk = nullptr) {
    const int n = j1 - j0;
    if (n <= 0) return;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // everyone is done with the previous unit's rings
#pragma unroll
    for (int q = 0; q < G::kLA; ++q) dma_a(q);
    if (GRAD) {
#pragma unroll
      for (int q = 0; q < G::kLB; ++q) dma_b(q);
    }
    bkt_init();
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

    GP g;  // G tile whose gradient GEMM is pending
    if constexpr (kPrefetch) {
      // A operands of the next logit GEMM read a step ahead (they fit in 32 registers per lane); one logit tile
      Op aop[KS];
      f32x16 z;  // logit tile whose epilogue is pending
      read_a(0, aop);
      top(0);
      int pb, pe;
      bkt_get(0, pb, pe);
      z = logits(aop, own);
      read_a(1, aop);
      epilogue(0, pb, pe, z, g, e_acc, posz, met, tk);
      // ring slots of iteration i, advanced without divisions: the A block loaded now, the B block loaded now,
      // the A block read now (step i+1) and the B block read now (step i-1)
      int sdA = (1 + G::kLA) % G::kNA, sdB = GRAD ? (1 + G::kLB) % G::kNB : 0, srA = 2 % G::kNA, srB = 0;
      for (int i = 1; i < n; ++i) {
        if (G::kK == 1 || i % G::kK == 0) barrier_at(i);
        dma_a(i + G::kLA, sdA);
        if (GRAD) dma_b(i + G::kLB, sdB);
        bkt_get(i, pb, pe);
        z = logits(aop, own);
        if (GRAD) grad_slot(srB, g, acc);
        read_slot(srA, aop);  // step n's slot holds a clamped copy of step n-1: harmless
        epilogue(i, pb, pe, z, g, e_acc, posz, met, tk);
        sdA = sdA + 1 == G::kNA ? 0 : sdA + 1;
        srA = srA + 1 == G::kNA ? 0 : srA + 1;
        if (GRAD) {
          sdB = sdB + 1 == G::kNB ? 0 : sdB + 1;
          srB = srB + 1 == G::kNB ? 0 : srB + 1;
        }
      }
    } else {
      // larger D: the logit GEMM of step i+1 runs in iteration i, reading its A operands from LDS right before
      // each MFMA; two logit tiles alternate roles
      f32x16 za = logits_lds(0, own), zb;
      int i = 0;
      for (; i + 1 < n; i += 2) {
        step_lds(i, own, za, zb, g, acc, e_acc, posz, met, tk);
        step_lds(i + 1, own, zb, za, g, acc, e_acc, posz, met, tk);
      }
      if (i < n) step_lds(i, own, za, zb, g, acc, e_acc, posz, met, tk);
    }
    // iteration n: the slot-packed block of step n-1 must have landed
    wait_vm_and_barrier<0>();
    if (GRAD) grad(n - 1, g, acc);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // Iteration i of the larger-D schedule: Z(i+1) into zn, gradient GEMM of step i-1, epilogue of step i (zc).
  __device__ inline void step_lds(int i, const Op* own, const f32x16& zc, f32x16& zn, GP& g, f32x16* acc,
                                  float& e_acc, float& posz, int* met, TopK<KT ? KT : 1>* tk) {
    top(i);
    int pb, pe;
    bkt_get(i, pb, pe);
    if (i + 1 < n_steps()) zn = logits_lds(i + 1, own);
    if (GRAD && i > 0) grad(i - 1, g, acc);
    epilogue(i, pb, pe, zc, g, e_acc, posz, met, tk);
  }
  __device__ inline int n_steps() const { return j1 - j0; }

  // Start of iteration i: the barrier (every kK iterations) and the loads of the iteration.
  __device__ inline void top(int i) {
    if (G::kK == 1 || i % G::kK == 0) barrier_at(i);
    dma_a(i + G::kLA);
    if (GRAD) dma_b(i + G::kLB);
  }

  __device__ inline void read_a(int i, Op* aop) const { read_slot(i % G::kNA, aop); }
  __device__ inline void read_slot(int slot, Op* aop) const {
    const char* a = lds + slot * G::kStepBytes;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) aop[ks] = lds_a<T, D>(a, lane % 32, ks, lane);
  }

  __device__ inline f32x16 logits(const Op* aop, const Op* own) const {
    f32x16 z = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) z = EL::mma(aop[ks], own[ks], z);
    return z;
  }
  __device__ inline f32x16 logits_lds(int i, const Op* own) const {
    const char* a = ringA(i);
    f32x16 z = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) z = EL::mma(lds_a<T, D>(a, lane % 32, ks, lane), own[ks], z);
    return z;
  }

  __device__ inline void grad(int j, const GP& g, f32x16* acc) const {
    grad_slot(j % (G::kNB ? G::kNB : 1), g, acc);
  }
  __device__ inline void grad_slot(int slot, const GP& g, f32x16* acc) const {
    const char* b = lds + (G::kNA + slot) * G::kStepBytes;
#pragma unroll
    for (int db = 0; db < NDBE; ++db)
#pragma unroll
      for (int q = 0; q < EL::kGroups; ++q) {
        if constexpr (F16G)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              g.op(q), *(const f16x8*)((const T*)b + slot_off<T>(D, DB0 + db, q, lane)), acc[db], 0, 0, 0);
        else
          acc[db] = EL::mma(g.op(q), lds_b<T, D>(b, DB0 + db, q, lane), acc[db]);
      }
  }

  // Epilogue of step j (called for j = 0, 1, ... in order): positives of the step (bucket [pb, pe)),
  // loss sums (FWD), the G tile (GRAD) and, with MET, the Cut Metrics counts of the lane: met[0] logits
  // predicted positive (z > 0), met[1] positives predicted positive, met[2] positives.
  __device__ inline void epilogue(int j, int pb, int pe, const f32x16& z, GP& g, float& e_acc, float& posz,
                                  int* met, TopK<KT ? KT : 1>* tk) {
    if constexpr (KT > 0) {
      // scoring: keep the lane's best items (real items only: V is padded to a multiple of 256, so up to 7
      // whole steps past V are swept, besides a ragged last one). Only the values above the lane's current k-th
      // best are inserted, one at a time, picked by a select chain (no dynamic register indexing). The lane's
      // bound lim (32-bit, V < 2^31) is 32 for steps wholly below V, the number of real items left in a step
      // holding V, and <= 0 -- nothing passes -- for steps at or beyond V.
      const float thr = tk->last();
      const int item0 = (j0 + j) * 32 + (lane / 32) * 4;
      const int lim = (int64_t)(j0 + j + 1) * 32 > nX ? (int)nX - item0 : 32;  // items of this lane below V
      uint32_t cand = 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i)  // item acc_pos(i, lane / 32)
        cand |= (z[i] > thr && (i / 4) * 8 + (i % 4) < lim) ? (1u << i) : 0u;
      while (cand) {
        const int i = __builtin_ctz(cand);
        cand &= cand - 1u;
        float x = z[0];
#pragma unroll
        for (int q = 1; q < 16; ++q) x = i == q ? z[q] : x;
        tk->template insert<true>(x, item0 + (i / 4) * 8 + (i % 4));
      }
      return;
    }
    float c[16];
    if (FWD)
      epi_rows<GRAD, false, LOSS>(z, 0u, c, e_acc, posz);
    else
      epi_items<false>(z, 0u, c);
    if (MET) {
#pragma unroll
      for (int i = 0; i < 16; ++i) met[0] += z[i] > 0.f ? 1 : 0;
    }
    if (pe > pb) {
      const uint32_t pm = positive_mask(pairs, pb, pe, own0, (j0 + j) * 32, FWD, lmask(), lane);
      if (pm) {
        if (apply_pos) {
#pragma unroll
          for (int q = 0; q < 16; ++q)
            if (pm & (1u << q)) {
              if (FWD) posz += z[q];
              c[q] -= 1.f;
            }
        }
        if (MET) {
          uint32_t gt = 0u;
#pragma unroll
          for (int q = 0; q < 16; ++q) gt |= (z[q] > 0.f ? 1u : 0u) << q;
          met[1] += __builtin_popcount(pm & gt);
          met[2] += __builtin_popcount(pm);
        }
      }
    }
    if (GRAD) g.set(c);
  }
};

// ---------------------------------------------------------------------------------------------------------
// Epilogue of one 32x32 logit tile (16 values per lane) as a fixed list of vector operations, so that the
// interleaved engine can hand out an equal share of them after each MFMA. The arithmetic is that of epi_rows
// (forward: w = 1 + e^-z, products over pairs and quads, one reciprocal per quad, log2 of the tile product) and
// of epi_items (backward: c = 1/(1 + e^-z) - 1/2), in the same association, so both engines give the same bits.
// ---------------------------------------------------------------------------------------------------------
template <typename GT>
struct EpiState {
  float w[16], w2[8], w4[4], r4[4], ra[4], rb[4];
  float p01, p23, wp, lg, e_inc;
  bool slow;
  GT g[2];  // G tile of the previous step, packed from its c by the kCvt operations
};

#ifndef CUTBCE_PRE_OPS
#define CUTBCE_PRE_OPS 0  // epilogue operations issued before the first MFMA of an iteration (with its first reads)
#endif
template <bool FWD, bool GRAD, int NSLOT, typename GT = bf16x8, int PRE_EXTRA = CUTBCE_PRE_OPS>
struct EpiOps {
  using State = EpiState<GT>;
  enum { kCvt = 0, kT, kE, kW, kM2, kM4, kR, kA, kB, kF, kWp, kLog, kEi, kCmp, kRc, kS };
  struct Tbl {
    short op[128];
    short start[34];
    int n, npre;
  };
  // Natural order: the first half of the previous step's G tile is packed before any MFMA (pre-slot), the second
  // half right after; then pairs of logits through exp, the pair and quad products, and each quad's batch
  // inversion one pair later (so the reciprocal's latency is covered); the tile product and its log come last.
  // (Packing after the iteration's branches instead, with the packed tile carried, measured 2.5% slower in the
  // forward sweep: there the conversions overlap no MFMA.)
  static constexpr Tbl make() {
    Tbl t{};
    int n = 0;
    auto push = [&](int kind, int arg) { t.op[n++] = (short)(kind * 64 + arg); };
    if (GRAD)
      for (int p = 0; p < 4; ++p) push(kCvt, p);
    int npre = n + PRE_EXTRA;
    for (int p = 0; p < 8; ++p) {
      push(kT, 2 * p);
      push(kT, 2 * p + 1);
      if (GRAD && p == 0)
        for (int q = 4; q < 8; ++q) push(kCvt, q);
      push(kE, 2 * p);
      push(kE, 2 * p + 1);
      push(kW, 2 * p);
      push(kW, 2 * p + 1);
      if (FWD) {
        push(kM2, p);
        if (p & 1) {
          push(kM4, p / 2);
          if (GRAD) push(kR, p / 2);
        }
        if (GRAD && p >= 2 && !(p & 1)) {
          const int q = p / 2 - 1;
          push(kA, q);
          push(kB, q);
          for (int j = 0; j < 4; ++j) push(kF, 4 * q + j);
        }
      } else {
        push(kRc, 2 * p);
        push(kRc, 2 * p + 1);
        push(kS, 2 * p);
        push(kS, 2 * p + 1);
      }
    }
    if (FWD) {
      if (GRAD) {
        push(kA, 3);
        push(kB, 3);
        for (int j = 0; j < 4; ++j) push(kF, 12 + j);
      }
      push(kWp, 0);
      push(kWp, 1);
      push(kWp, 2);
      push(kLog, 0);
      push(kEi, 0);
      push(kCmp, 0);
    }
    t.n = n;
    t.npre = npre < n ? npre : n;
    for (int j = 0; j <= NSLOT; ++j) t.start[j] = (short)(t.npre + (n - t.npre) * j / (NSLOT > 0 ? NSLOT : 1));
    return t;
  }
  static constexpr Tbl tbl = make();

  template <int OPC>
  __device__ static inline void op(const f32x16& z, float* c, State& s) {
    constexpr int kind = OPC / 64, a = OPC % 64;
    if constexpr (kind == kCvt) {
      using E = typename std::conditional<std::is_same<GT, f16x8>::value, _Float16, __bf16>::type;
      s.g[a / 4][2 * (a % 4)] = (E)c[2 * a];
      s.g[a / 4][2 * (a % 4) + 1] = (E)c[2 * a + 1];
    } else if constexpr (kind == kT) {
      s.w[a] = z[a] * -kLog2e;
    } else if constexpr (kind == kE) {
      s.w[a] = __builtin_amdgcn_exp2f(s.w[a]);
    } else if constexpr (kind == kW) {
      s.w[a] = 1.f + s.w[a];
    } else if constexpr (kind == kM2) {
      s.w2[a] = s.w[2 * a] * s.w[2 * a + 1];
    } else if constexpr (kind == kM4) {
      s.w4[a] = s.w2[2 * a] * s.w2[2 * a + 1];
    } else if constexpr (kind == kR) {
      s.r4[a] = __builtin_amdgcn_rcpf(s.w4[a]);
    } else if constexpr (kind == kA) {
      s.ra[a] = s.r4[a] * s.w2[2 * a + 1];
    } else if constexpr (kind == kB) {
      s.rb[a] = s.r4[a] * s.w2[2 * a];
    } else if constexpr (kind == kF) {
      // c[4q] = ra w[4q+1], c[4q+1] = ra w[4q], c[4q+2] = rb w[4q+3], c[4q+3] = rb w[4q+2]  (minus 1/2)
      c[a] = ((a % 4) < 2 ? s.ra[a / 4] : s.rb[a / 4]) * s.w[a ^ 1] - 0.5f;
    } else if constexpr (kind == kWp) {
      if constexpr (a == 0) s.p01 = s.w4[0] * s.w4[1];
      else if constexpr (a == 1) s.p23 = s.w4[2] * s.w4[3];
      else s.wp = s.p01 * s.p23;
    } else if constexpr (kind == kLog) {
      s.lg = __builtin_amdgcn_logf(s.wp);
    } else if constexpr (kind == kEi) {
      s.e_inc = kLn2 * (s.lg - 16.f);
    } else if constexpr (kind == kCmp) {
      s.slow = !(s.wp <= kFastProd);
    } else if constexpr (kind == kRc) {
      s.w[a] = __builtin_amdgcn_rcpf(s.w[a]);
    } else if constexpr (kind == kS) {
      c[a] = s.w[a] - 0.5f;
    }
  }
  template <int I, int E>
  __device__ static inline void ops(const f32x16& z, float* c, State& s) {
    if constexpr (I < E) {
      op<tbl.op[I]>(z, c, s);
      ops<I + 1, E>(z, c, s);
    }
  }
  __device__ static inline void pre(const f32x16& z, float* c, State& s) { ops<0, tbl.npre>(z, c, s); }
  template <int J>
  __device__ static inline void slot(const f32x16& z, float* c, State& s) {
    ops<tbl.start[J], tbl.start[J + 1]>(z, c, s);
  }
  __device__ static inline void all(const f32x16& z, float* c, State& s) { ops<0, tbl.n>(z, c, s); }
};

// ---------------------------------------------------------------------------------------------------------
// Polynomial epilogue of the dE sweep for tiles whose logits are known to satisfy |z| <= 1 (the sweep checks the
// Cauchy-Schwarz bound |H[r].E[v]| <= ||H[r]|| ||E[v]|| per wave): c = sigma(z) - 1/2 = tanh(z/2)/2 as the
// Taylor polynomial z/4 - z^3/48 + z^5/480 - 17 z^7/80640 (an alternating series: the error is below the first
// omitted term 31 |z|^9 / 1451520 <= 2.2e-5, relative 1e-4 at |z| = 1 and smaller below), evaluated on packed
// f16 pairs. It needs no transcendental and writes the f16 G operand directly; its f16 rounding (about 2^-10
// relative) is finer than the bf16 G of the exact path.
// ---------------------------------------------------------------------------------------------------------
struct PolyState {
  f16x2 zh[8], z2[8], t[8];
};
// Largest ||H[r]|| ||E[v]|| (over a wave's items and all rows) for which the polynomial is used; the margin below
// 1 covers the float32 rounding of the norms and of the logit itself.
constexpr float kPolyBound = 0.999f;

template <int NSLOT>
struct EpiPoly {
  enum { kCz = 1, kZ2, kP3, kP2, kP1, kC };
  struct Tbl {
    short op[64];
    short start[34];
    int n;
  };
  static constexpr Tbl make() {
    Tbl t{};
    int n = 0;
    auto push = [&](int kind, int arg) { t.op[n++] = (short)(kind * 64 + arg); };
    for (int p = 0; p < 8; p += 2)
      for (int kind = kCz; kind <= kC; ++kind) {
        push(kind, p);
        push(kind, p + 1);
      }
    t.n = n;
    for (int j = 0; j <= NSLOT; ++j) t.start[j] = (short)(n * j / (NSLOT > 0 ? NSLOT : 1));
    return t;
  }
  static constexpr Tbl tbl = make();

  template <int OPC>
  __device__ static inline void op(const f32x16& z, PolyState& s, f16x8* gn) {
    constexpr int kind = OPC / 64, a = OPC % 64;
    const f16x2 c3 = {(_Float16)(-17.0 / 80640.0), (_Float16)(-17.0 / 80640.0)};
    const f16x2 c2 = {(_Float16)(1.0 / 480.0), (_Float16)(1.0 / 480.0)};
    const f16x2 c1 = {(_Float16)(-1.0 / 48.0), (_Float16)(-1.0 / 48.0)};
    const f16x2 c0 = {(_Float16)0.25, (_Float16)0.25};
    if constexpr (kind == kCz) {
      s.zh[a] = f16x2{(_Float16)z[2 * a], (_Float16)z[2 * a + 1]};
    } else if constexpr (kind == kZ2) {
      s.z2[a] = s.zh[a] * s.zh[a];
    } else if constexpr (kind == kP3) {
      s.t[a] = s.z2[a] * c3 + c2;
    } else if constexpr (kind == kP2) {
      s.t[a] = s.z2[a] * s.t[a] + c1;
    } else if constexpr (kind == kP1) {
      s.t[a] = s.z2[a] * s.t[a] + c0;
    } else if constexpr (kind == kC) {
      const f16x2 c = s.zh[a] * s.t[a];
      gn[a / 4][2 * (a % 4)] = c[0];
      gn[a / 4][2 * (a % 4) + 1] = c[1];
    }
  }
  template <int I, int E>
  __device__ static inline void ops(const f32x16& z, PolyState& s, f16x8* gn) {
    if constexpr (I < E) {
      op<tbl.op[I]>(z, s, gn);
      ops<I + 1, E>(z, s, gn);
    }
  }
  template <int J>
  __device__ static inline void slot(const f32x16& z, PolyState& s, f16x8* gn) {
    ops<tbl.start[J], tbl.start[J + 1]>(z, s, gn);
  }
  __device__ static inline void all(const f32x16& z, PolyState& s, f16x8* gn) { ops<0, tbl.n>(z, s, gn); }
};

// ---------------------------------------------------------------------------------------------------------
// Polynomial epilogue of the forward sweep for waves whose logits all satisfy |z| <= B (the sweep checks
// max_r ||H[r]|| over the wave's rows times max_v ||E[v]||, a Cauchy-Schwarz bound). Per logit it needs the loss
// term of the signed form, log(1 + e^-z) - ln 2 = -z/2 + log cosh(z/2), and c = sigma(z) - 1/2 = tanh(z/2)/2:
//   log cosh(z/2) = u/8 - u^2/192 + u^3/2880 - 17 u^4/645120 + ...   (u = z^2),
//   tanh(z/2)/2   = z (1/4 - u/48 + u^2/480 - 17 u^3/80640 + 31 u^4/1451520 - ...).
// Both are alternating series with decreasing terms for |z| <= 1, so the error is below the first omitted term.
// Long form (B = 0.8): loss through u^3, c through u^3: errors below 4.4e-6 per loss term (1.4e-5 of the smallest
// possible BCE term, softplus(-1) > 0.31) and 2.9e-6 on c. Short form (B = 0.45): loss through u^2, c through
// u^2: errors below 3.2e-6 per loss term and 3.2e-6 on c, two operations less per pair of logits. The arithmetic
// runs on packed f16 pairs (z rounded once to f16, relative 2^-11); the log cosh terms are summed in fp32 by
// v_dot2_f32_f16 (exact f16 products) into kPolyAcc accumulators carried over the unit's steps (pair a feeds
// accumulator a % kPolyAcc: short dependent chains), and c is written straight into the f16 G tile. The -z/2
// terms are not summed here: over a row's items they add up to the rank-1 -H[r].sum_v E[v] / 2, which the finish
// adds in float64 for the rows flagged as polynomial. (Measured: a dot product per pair for -z/2 in one chain
// with the rest cost the sweep 5%; two accumulators reset every step 0.6% against four carried ones.)
// ---------------------------------------------------------------------------------------------------------
constexpr float kPolyBoundF = 0.8f;       // long form
constexpr float kPolyBoundShort = 0.45f;  // short form
#ifndef CUTBCE_POLY_ACC
#define CUTBCE_POLY_ACC 4
#endif
constexpr int kPolyAcc = CUTBCE_POLY_ACC;  // independent loss accumulators (pairs a, a + kPolyAcc, ... share one)
struct PolyStateF {
  f16x2 zh[8], u[8], t[8], l[8];
  float e[kPolyAcc];  // the sweep's log cosh terms so far, carried across steps
};

template <int NSLOT, bool SHORT>
struct EpiPolyF {
  enum { kCz = 1, kZ2, kP3, kP2, kP1, kC, kL2, kL1, kLa };
  struct Tbl {
    short op[80];
    short start[34];
    int n;
  };
  // groups of four logit pairs through every stage, so that each dependent operation comes three independent
  // ones after its input (two pairs per group measured 1.3% slower at D = 128, 2.5% at D = 64; the dE sweep's
  // polynomial keeps groups of two, which measured 0.7% faster there)
  static constexpr Tbl make() {
    Tbl t{};
    int n = 0;
    auto push = [&](int kind, int arg) { t.op[n++] = (short)(kind * 64 + arg); };
    for (int p = 0; p < 8; p += 4)
      for (int kind = kCz; kind <= kLa; ++kind) {
        if (SHORT && (kind == kP3 || kind == kL2)) continue;
        for (int q = 0; q < 4; ++q) push(kind, p + q);
      }
    t.n = n;
    for (int j = 0; j <= NSLOT; ++j) t.start[j] = (short)(n * j / (NSLOT > 0 ? NSLOT : 1));
    return t;
  }
  static constexpr Tbl tbl = make();
  typedef __fp16 h2 __attribute__((ext_vector_type(2)));

  // Each result is tied to an empty asm statement where it is computed: otherwise the optimiser moves this pure
  // arithmetic out of its MFMA slot (measured: the loss sums of all six unrolled iterations sunk into the last
  // one, other stages hoisted in front of the first MFMA), which leaves the MFMAs without vector work beside them.
  template <typename X>
  __device__ static inline void pin(X& x) {
    asm volatile("" : "+v"(x));
  }
  template <int OPC>
  __device__ static inline void op(const f32x16& z, PolyStateF& s, f16x8* gn) {
    constexpr int kind = OPC / 64, a = OPC % 64;
    const f16x2 c3 = {(_Float16)(-17.0 / 80640.0), (_Float16)(-17.0 / 80640.0)};
    const f16x2 c2 = {(_Float16)(1.0 / 480.0), (_Float16)(1.0 / 480.0)};
    const f16x2 c1 = {(_Float16)(-1.0 / 48.0), (_Float16)(-1.0 / 48.0)};
    const f16x2 c0 = {(_Float16)0.25, (_Float16)0.25};
    const f16x2 b3 = {(_Float16)(1.0 / 2880.0), (_Float16)(1.0 / 2880.0)};
    const f16x2 b2 = {(_Float16)(-1.0 / 192.0), (_Float16)(-1.0 / 192.0)};
    const f16x2 b1 = {(_Float16)0.125, (_Float16)0.125};
    if constexpr (kind == kCz) {
      s.zh[a] = f16x2{(_Float16)z[2 * a], (_Float16)z[2 * a + 1]};
      pin(s.zh[a]);
    } else if constexpr (kind == kZ2) {
      s.u[a] = s.zh[a] * s.zh[a];
      pin(s.u[a]);
    } else if constexpr (kind == kP3) {
      s.t[a] = s.u[a] * c3 + c2;
      pin(s.t[a]);
    } else if constexpr (kind == kP2) {
      s.t[a] = s.u[a] * (SHORT ? c2 : s.t[a]) + c1;
      pin(s.t[a]);
    } else if constexpr (kind == kP1) {
      s.t[a] = s.u[a] * s.t[a] + c0;
      pin(s.t[a]);
    } else if constexpr (kind == kC) {
      f16x2 c = s.zh[a] * s.t[a];
      pin(c);
      gn[a / 4][2 * (a % 4)] = c[0];
      gn[a / 4][2 * (a % 4) + 1] = c[1];
    } else if constexpr (kind == kL2) {
      s.l[a] = s.u[a] * b3 + b2;
      pin(s.l[a]);
    } else if constexpr (kind == kL1) {
      s.l[a] = s.u[a] * (SHORT ? b2 : s.l[a]) + b1;
      pin(s.l[a]);
    } else if constexpr (kind == kLa) {  // + u (1/8 - u/192 + u^2/2880) for both logits
      constexpr int q = a % kPolyAcc;
      s.e[q] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, s.l[a]), __builtin_bit_cast(h2, s.u[a]), s.e[q], false);
      pin(s.e[q]);
    }
  }
  template <int I, int E>
  __device__ static inline void ops(const f32x16& z, PolyStateF& s, f16x8* gn) {
    if constexpr (I < E) {
      op<tbl.op[I]>(z, s, gn);
      ops<I + 1, E>(z, s, gn);
    }
  }
  template <int J>
  __device__ static inline void slot(const f32x16& z, PolyStateF& s, f16x8* gn) {
    ops<tbl.start[J], tbl.start[J + 1]>(z, s, gn);
  }
  __device__ static inline void all(const f32x16& z, PolyStateF& s, f16x8* gn) { ops<0, tbl.n>(z, s, gn); }
};

// ---------------------------------------------------------------------------------------------------------
// Interleaved step engine for bf16 operands with D <= 128 (8 waves per workgroup, two per SIMD).
//
// With two waves per SIMD the matrix pipe accepts MFMAs from both, so the sweep runs at the MFMA rate only if
// each wave keeps issuing MFMAs while it does its vector work. Iteration i of a wave therefore issues three
// mutually independent pieces of work and lets them interleave (the order is pinned with scheduling groups):
//   - the logit GEMM of step i+1 (A operands read from LDS inside the iteration),
//   - the gradient GEMM of step i-1 (its G tile packed to bf16 at the start of the iteration),
//   - the epilogue of step i on the vector ALU, whose logits came from iteration i-1.
// The loop is unrolled by the ring length (6), so every ring slot and barrier position is a constant: LDS
// reads use immediate offsets from per-lane base addresses, and the scalar work per iteration is one offset
// update and the two DMA destinations. Rare work (the |z| form of the forward epilogue, positives of the
// step) runs in branches after the interleaved block.
//
// Rings: the d-packed block of step j (A) is loaded at iteration j - LA into slot j % 6 and read in iteration
// j - 1; the slot-packed block (B) is loaded at iteration j - LB and read in iteration j + 1. A barrier opens
// every even iteration and waits for all ring loads but those of the two iterations before it. Then (K = 2
// iterations per barrier, two iterations of loads in flight): LA >= K + 3 and LB >= K + 1 make every block
// land before a barrier that precedes its reads, and 6 >= LA + K - 1, 6 >= LB + K + 1 put a barrier between
// the last read of a slot and its refill. (Reading an iteration's first operands at the end of the one before,
// with 8-slot rings, measured 1.5% slower.)
// Streamed blocks are addressed through buffer descriptors rebased every 64 steps (offsets stay small for
// any vocabulary); loads past the end of an array return zeros, whose logits add nothing (z = 0 gives a zero
// loss term in the signed form and c = 0).
// ---------------------------------------------------------------------------------------------------------
// F16G: the gradient GEMM runs on f16 operands (G and the slot-packed rows, which the H preparation stores as
// f16 scaled by a power of two); used by the dE sweep, whose tiles can then take the polynomial epilogue.
// POS: the sweep takes positives from the buckets (the dE sweep; the forward only when its positives are not
// gathered by the finish). Without them the bucket pointers are never read.
template <int D, bool FWD, bool GRAD, bool F16G = false, bool POS = !FWD || !kGatherPositives>
struct Pipe {
  static constexpr int NW = 8, KS = D / 16, NDB = D / 32;
  using GOp = typename std::conditional<F16G, f16x8, bf16x8>::type;  // operands of the gradient GEMM
  __device__ static inline f32x16 mma_g(GOp a, GOp b, f32x16 c) {
    if constexpr (F16G)
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static constexpr int SB = 32 * D * 2;  // bytes of a 32-row block
  static constexpr int CPR = D / 8;      // 16-byte chunks per d-packed row
  static constexpr int K = 2, NR = 6, LA = 5, LB = 3;
  static constexpr int LOADB = SB / NW >= 1024 ? 16 : 4;  // bytes per lane per DMA instruction
  static constexpr int WB = 64 * LOADB;
  static constexpr int NLD = SB / WB / NW;  // DMA instructions per wave and block
  static constexpr int NRING = GRAD ? 2 : 1;
  static constexpr int INFL = 2 * NLD * NRING;  // ring loads a barrier leaves in flight (two iterations)
  static constexpr int RING_B = NR * SB;
  static constexpr int BKT = NRING * NR * SB;        // bucket pointers of two 64-step blocks (2 x 128 ints)
  static constexpr int LMASK = BKT + 2 * 128 * 4;     // per-wave positive masks (64 ints each)
  static constexpr int LDS_BYTES = LMASK + NW * 256;
  static_assert(NLD >= 1 && SB % (WB * NW) == 0, "DMA split");
  static_assert(LA >= K + 3 && NR >= LA + K - 1 && LB >= K + 1 && NR >= LB + K + 1, "ring constraints");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

  char* lds;
  uint32_t lds_s;  // LDS byte address of `lds`, wave-uniform
  int wave, lane;
  const char* X;     // d-packed streamed operand (E in the forward, Hc in the backward)
  int64_t x_bytes;   // its size in bytes
  const char* Xsp;   // slot-packed copy (Evp / Hrp)
  int64_t xsp_bytes;
  const int32_t* bptr;
  const int2* pairs;
  int64_t bbase;
  int own0, j0, j1;
  uint32_t aoff[KS];  // per-lane LDS byte offset of A chunk ks inside slot 0
  uint32_t boff;      // per-lane LDS byte offset of the B operand inside slot 0 of the B ring
  uint32_t voffA[NLD], voffB[NLD];
  __amdgpu_buffer_rsrc_t rA, rB;
  int soff;
  uint64_t nem;  // steps of the current 64-step block whose bucket of positives is not empty

  __device__ inline void setup(char* l, int w, int ln) {
    lds = l;
    wave = __builtin_amdgcn_readfirstlane(w);
    lane = ln;
    lds_s = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_void*)l);
    const int r = ln % 32, h = ln / 32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) aoff[ks] = r * (D * 2) + (((2 * ks + h) ^ swz<CPR>(r)) * 16);
    boff = RING_B + ln * 16;
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int inst = wave + q * NW;
      const int pos = inst * WB + ln * LOADB;
      const int row = pos / (D * 2), within = pos % (D * 2);
      voffA[q] = row * (D * 2) + (((within / 16) ^ swz<CPR>(row)) * 16) + within % 16;
      voffB[q] = pos;
    }
  }
  __device__ static inline __amdgpu_buffer_rsrc_t rsrc(const char* base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, n, 0x00020000);
  }
  // descriptors for the loads of iterations 64b .. 64b + 63 (soffset = (i - 64b) * SB)
  __device__ inline void window(int b) {
    const int64_t a0 = ((int64_t)j0 + 64 * b + LA) * SB, b0 = ((int64_t)j0 + 64 * b + LB) * SB;
    rA = rsrc(X + a0, x_bytes - a0);
    if (GRAD) rB = rsrc(Xsp + b0, xsp_bytes - b0);
    soff = 0;
  }
  __device__ inline void dma(__amdgpu_buffer_rsrc_t r, uint32_t ring, int slot, const uint32_t* voff, int so) const {
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      lds_void* dst = (lds_void*)(size_t)(lds_s + ring + slot * SB + (wave + q * NW) * WB);
      if constexpr (LOADB == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff[q], so, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, voff[q], so, 0, 0);
    }
  }
  // the loads of iteration i (after the barrier of the iteration, if any)
  __device__ inline void dma_iter(int sAw, int sBw) {
    dma(rA, 0, sAw, voffA, soff);
    if (GRAD) dma(rB, RING_B, sBw, voffB, soff);
    soff += SB;
  }

  // Bucket pointers of block b (steps 64b .. 64b + 63 of the unit: entries j0 + 64b .. j0 + 64b + 64 of bptr,
  // the last step's end included) go to LDS buffer b & 1 by DMA (waves 0 and 1, 64 entries each; entries past
  // the unit's end j1 read as 0 and are never used). A block is loaded 64 steps before it is needed, so no
  // register waits for the load.
  __device__ inline void bkt_dma(int b) const {
    if (POS && wave < 2) {
      const int64_t first = (int64_t)j0 + 64 * b + 64 * wave;
      const int64_t cnt = (int64_t)j1 + 1 - first;
      const __amdgpu_buffer_rsrc_t r = rsrc((const char*)(bptr + bbase + first), cnt * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(size_t)(lds_s + BKT + (b & 1) * 512 + wave * 256), 4,
                                               lane * 4, 0, 0, 0);
    }
  }
  __device__ inline const int* bkt(int b) const { return (const int*)(lds + BKT) + (b & 1) * 128; }
  // At iteration 64b (a barrier iteration, after the barrier): block b is current and the load window moves.
  __device__ inline void block_start(int b) {
    if (POS) {
      const int* k = bkt(b);
      nem = __builtin_amdgcn_ballot_w64(k[lane] != k[lane + 1]);
    } else {
      nem = 0;
    }
    window(b);
  }

  __device__ inline bf16x8 rdA(int slot, int ks) const { return *(const bf16x8*)(lds + aoff[ks] + slot * SB); }
  __device__ inline GOp rdB(int slot, int m) const { return *(const GOp*)(lds + boff + slot * SB + m * 1024); }

  __device__ inline f32x16 logits(int slot, const bf16x8* own) const {
    f32x16 z = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rdA(slot, ks), own[ks], z, 0, 0, 0);
    return z;
  }

  __device__ inline uint32_t step_mask(int i) {
    const int* k = bkt(i >> 6);
    const int pb = __builtin_amdgcn_readfirstlane(k[i & 63]), pe = __builtin_amdgcn_readfirstlane(k[(i & 63) + 1]);
    uint32_t* lm = (uint32_t*)(lds + LMASK) + wave * 64;
    return positive_mask(pairs, pb, pe, own0, (j0 + i) * 32, FWD, lm, lane);
  }
  // positives of step i on a packed f16 G tile: 1 subtracted at each positive
  __device__ inline void positives_f16(int i, f16x8* g) {
    const uint32_t pm = step_mask(i);
    if (pm) {
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (pm & (1u << q)) g[q / 8][q % 8] -= (_Float16)1.0f;
    }
  }
  // positives of step i (its bucket is not empty): mask, then c -= 1 there and (forward) posz += z
  __device__ inline void positives(int i, const f32x16& z, float* c, float& posz) {
    const uint32_t pm = step_mask(i);
    if (pm) {
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (pm & (1u << q)) {
          if (FWD) posz += z[q];
          c[q] -= 1.f;
        }
    }
  }

  // MFMAs of an interleaved iteration: with the gradient GEMM, even j = logit MFMA j/2 of step i+1 and odd
  // j = gradient MFMA (j-1)/2 of step i-1 (tile (j-1)/4, G half ((j-1)/2) % 2); without it, logit MFMA j.
  static constexpr int NM = GRAD ? 2 * KS : KS;
#ifndef CUTBCE_READ_AHEAD
#define CUTBCE_READ_AHEAD 3
#endif
  static constexpr int RA = CUTBCE_READ_AHEAD;  // MFMAs between an operand's LDS read and its use
  using ES = EpiOps<FWD, GRAD, NM, GOp>;
  static_assert(!GRAD || KS == 2 * NDB, "logit and gradient MFMAs alternate");

  // gradient MFMA k of an iteration takes chunk gm(k): d-blocks in turn, first every d-block's first G half, then
  // the second halves, so that MFMAs accumulating into one tile are NDB gradient MFMAs apart
  static constexpr int gm(int k) { return (k % NDB) * 2 + k / NDB; }
  __device__ inline bf16x8 opnd_read(int j, int sAr, int sBr) const {
    return GRAD ? ((j & 1) ? __builtin_bit_cast(bf16x8, rdB(sBr, gm(j >> 1))) : rdA(sAr, j >> 1)) : rdA(sAr, j);
  }
  // Slot J: MFMA J, its share of the epilogue, and the LDS read of the operand of MFMA J + RA. sched_barrier
  // keeps the slots in order (the compiler would otherwise issue each read right before its MFMA).
  // POLY 1 / 2: the polynomial epilogue (2: the forward's short form; writes the next G tile gn; the gradient
  // MFMAs use the carried g) instead of
  // the exact one (packs the carried c of the previous step into st.g for the gradient MFMAs, writes the new c).
  template <int J, int POLY>
  __device__ inline void slots(int sAr, int sBr, const bf16x8* own, f32x16* acc, f32x16& zn, const f32x16& zc,
                               float* c, typename ES::State& st, PolyState& ps, PolyStateF& psf, const GOp* g,
                               GOp* gn, bf16x8* opnd) const {
    if constexpr (J < NM) {
      if constexpr (GRAD && (J & 1))
        acc[gm(J >> 1) >> 1] = mma_g((POLY ? g : st.g)[gm(J >> 1) & 1], __builtin_bit_cast(GOp, opnd[J]),
                                     acc[gm(J >> 1) >> 1]);
      else
        zn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[J], own[GRAD ? J >> 1 : J], zn, 0, 0, 0);
      if constexpr (POLY && FWD)
        EpiPolyF<NM, POLY == 2>::template slot<J>(zc, psf, gn);
      else if constexpr (POLY)
        EpiPoly<NM>::template slot<J>(zc, ps, gn);
      else
        ES::template slot<J>(zc, c, st);
      if constexpr (J + RA < NM) opnd[J + RA] = opnd_read(J + RA, sAr, sBr);
      __builtin_amdgcn_sched_barrier(0);
      slots<J + 1, POLY>(sAr, sBr, own, acc, zn, zc, c, st, ps, psf, g, gn, opnd);
    }
  }

  // One iteration (see the struct comment). HASG: the gradient GEMM of step i-1 is due (every iteration but
  // the first). Slots: sAr / sBr read, sAw / sBw loaded.
  __device__ static inline void pack(const float* c, GOp* g) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if constexpr (F16G)
          g[q][jj] = (_Float16)c[q * 8 + jj];
        else
          g[q][jj] = (__bf16)c[q * 8 + jj];
      }
  }

  // The previous step's G tile is carried in c (exact epilogue: float values, packed inside the iteration) or in
  // g (polynomial epilogue: packed f16); on return they hold step i's.
  // POLY (F16G sweeps): the polynomial epilogue (EpiPoly in the dE sweep, EpiPolyF in the forward).
  template <bool HASG, int POLY>
  __device__ inline void iter(int i, int sAr, int sBr, int sAw, int sBw, bool bar, const bf16x8* own,
                              f32x16* acc, f32x16& zc, float* c, GOp* g, float& e_acc, float& posz,
                              PolyStateF& psf) {
    static_assert(!POLY || (F16G && GRAD && !(FWD && POS)), "polynomial epilogue: f16 sweeps (forward: gathered positives)");
    static_assert(POLY != 2 || FWD, "short polynomial: forward only");
    const bool newblk = bar && (i & 63) == 0;
    if (bar) {
      wait_vm_and_barrier<INFL>();
      if (newblk) block_start(i >> 6);
    }
    dma_iter(sAw, sBw);
    if (newblk) bkt_dma((i >> 6) + 1);  // after the ring loads: the next barrier waits for nothing extra
    typename ES::State st;
    PolyState ps;
    GOp gn[2];
    f32x16 zn;
    if constexpr (HASG || !GRAD) {
      bf16x8 opnd[NM];
#pragma unroll
      for (int j = 0; j < RA; ++j) opnd[j] = opnd_read(j, sAr, sBr);
      if constexpr (!POLY) ES::pre(zc, c, st);
      zn = f32x16{};
      __builtin_amdgcn_sched_barrier(0);
      slots<0, POLY>(sAr, sBr, own, acc, zn, zc, c, st, ps, psf, g, gn, opnd);
    } else {
      zn = logits(sAr, own);
      if constexpr (POLY && FWD)
        EpiPolyF<NM, POLY == 2>::all(zc, psf, gn);
      else if constexpr (POLY)
        EpiPoly<NM>::all(zc, ps, gn);
      else
        ES::all(zc, c, st);
    }
    if constexpr (POLY) {
      if (POS && __builtin_expect((nem >> (i & 63)) & 1, 0)) positives_f16(i, gn);
      g[0] = gn[0];
      g[1] = gn[1];
      zc = zn;
      return;
    }
    if (FWD) {
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(st.slow) != 0, 0)) {
        float dummy = 0.f;
        st.e_inc = 0.f;
        epi_rows<GRAD, false, true>(zc, 0u, c, st.e_inc, dummy);
      }
      e_acc += st.e_inc;
    }
    if (POS && __builtin_expect((nem >> (i & 63)) & 1, 0)) positives(i, zc, c, posz);
    zc = zn;
  }

  // Runs the steps [j0, j1) of a unit. own: owner operand; acc: gradient tiles; e_acc / posz: forward row sums.
  template <int POLY = 0>
  __device__ inline void run(const bf16x8* own, f32x16* acc, float& e_acc, float& posz) {
    const int n = j1 - j0;
    if (n <= 0) return;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // the previous unit's reads are done
    {
      const int64_t a0 = (int64_t)j0 * SB;
      const __amdgpu_buffer_rsrc_t r0 = rsrc(X + a0, x_bytes - a0);
#pragma unroll
      for (int q = 0; q < LA; ++q) dma(r0, 0, q, voffA, q * SB);
      if (GRAD) {
        const __amdgpu_buffer_rsrc_t r1 = rsrc(Xsp + a0, xsp_bytes - a0);
#pragma unroll
        for (int q = 0; q < LB; ++q) dma(r1, RING_B, q, voffB, q * SB);
      }
    }
    bkt_dma(0);
    bkt_dma(1);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    block_start(0);
    f32x16 zc = logits(0, own);
    // Step 0's A slot is refilled (step NR) by the loads of iteration 1, and neither iteration 0 nor 1 opens a
    // barrier: every wave's reads of it must be done before any wave gets there. Without this barrier a wave
    // that ran an iteration ahead (measured: on a kernel's first, cold launch) overwrote the block under a
    // wave still reading it, changing a few logits of that wave's rows.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float c[16];  // G tile of the last epilogue (exact epilogue)
    GOp g[2];     // the same, packed (polynomial epilogue)
    PolyStateF psf;  // the forward polynomial's loss accumulators (carried over the unit's steps)
#pragma unroll
    for (int q = 0; q < kPolyAcc; ++q) psf.e[q] = 0.f;
    // iteration 0: logits of step 1, epilogue of step 0 (no gradient yet); with the barrier above it counts
    // as a barrier iteration (the one before the loop)
    iter<false, POLY>(0, 1, 0, LA % NR, LB % NR, false, own, acc, zc, c, g, e_acc, posz, psf);
    int i = 1;
    // iterations 1 + 6m + u: slots A read (2 + u) % 6, B read u, A load u, B load (4 + u) % 6; barrier at odd u
    for (; i + NR - 1 < n; i += NR) {
#pragma unroll
      for (int u = 0; u < NR; ++u)
        iter<true, POLY>(i + u, (2 + u) % NR, u, (1 + LA + u) % NR, (1 + LB + u) % NR, (u & 1) != 0, own, acc, zc, c,
                         g, e_acc, posz, psf);
    }
    for (; i < n; ++i)
      iter<true, POLY>(i, (i + 1) % NR, (i - 1) % NR, (i + LA) % NR, (i + LB) % NR, (i & 1) == 0, own, acc, zc, c, g,
                       e_acc, posz, psf);
    // iteration n: the gradient GEMM of step n - 1
    wait_vm_and_barrier<0>();
    if (GRAD) {
      if constexpr (!POLY) pack(c, g);
      const int s = (n - 1) % NR;
#pragma unroll
      for (int m = 0; m < 2 * NDB; ++m) acc[m / 2] = mma_g(g[m % 2], rdB(s, m), acc[m / 2]);
    }
    if constexpr (POLY && FWD) {
      float et = psf.e[0];
#pragma unroll
      for (int q = 1; q < kPolyAcc; ++q) et += psf.e[q];
      e_acc += et;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
};

// Whether a sweep instance runs on the interleaved engine (bf16, D = 64 or 128, 8 waves, one pass, no Cut
// Metrics, no scoring) or on the general one.
template <typename T, int D, int NW, bool MET, int KT, int PART>
__host__ __device__ constexpr bool use_pipe() {
  return sizeof(T) == 2 && (D == 64 || D == 128) && NW == 8 && !MET && KT == 0 && PART == 0;
}
template <typename T, int D, int NW, bool FWD, bool GRAD, bool MET, int KT, int PART>
constexpr size_t sweep_lds() {
  if constexpr (use_pipe<T, D, NW, MET, KT, PART>())
    return Pipe<D <= 128 ? D : 128, FWD, GRAD, !FWD>::LDS_BYTES;
  else
    return Geo<T, D, NW, GRAD>::kLdsBytes;
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
  int4* metpart;   // [units][RW]: Cut Metrics counts (predicted positive, true positive, positives)
  bool pos_apply;  // positives enter the tiles (c - 1, the loss's sum of their logits); false: counted only
  uint8_t* rowform;  // [R_pad] (bf16, D <= 128): 1 where the row's waves took the polynomial epilogue, else 0
  float* topv;     // [units][RW][KT]: per-split top-KT logits (scoring)
  int32_t* topi;   // [units][RW][KT]: their item ids
};

// ---------------------------------------------------------------------------------------------------------
// Forward sweep. Persistent: gridDim.x workgroups (as many as can be resident, a multiple of 8); units (split s,
// row tile t) are assigned in contiguous per-XCD ranges so that the workgroups sharing an L2 stream the same
// part of E. With KT > 0 it scores instead: per-lane top-KT lists, merged per row and written per unit.
// ---------------------------------------------------------------------------------------------------------
// DHPART 0: one pass (loss, dH and optional Cut Metrics); 1 / 2: the first / second of two passes, each
// accumulating half of dH's d-blocks (half the accumulator registers, for f32 D = 256); the loss and the Cut
// Metrics come from pass 1.
template <typename T, int D, int NW, bool WITH_DH, bool MET, int KT, int DHPART = 0>
__global__ void __launch_bounds__(NW * 64) k_rows(RowsArgs a) {
  using EL = Elem<T>;
  constexpr int NDB = D / 32, NDBE = DHPART ? NDB / 2 : NDB, DB0 = DHPART == 2 ? NDB / 2 : 0;
  // bf16, D <= 128: the gradient GEMM takes f16 G tiles and the f16 Evp (scaled by 2^s; dH partials unscaled
  // when written)
  constexpr bool kF16 = std::is_same<T, __bf16>::value && evp_is_f16(1, D) && WITH_DH;
  using EN = Engine<T, D, NW, true, WITH_DH, MET, KT, DB0, NDBE, DHPART != 2, kF16>;
  constexpr int RW = NW * 32, KS = D / EL::kK;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
  const T* __restrict__ Hc = (const T*)a.Hc;

  const int n_valid = a.ctl->n_valid;
  const int Tt = (n_valid + RW - 1) / RW;
  if (Tt == 0) return;
  const int n_steps = (int)(a.V_pad / 32);
  const int P = gridDim.x;
  const int S = choose_splits(Tt, n_steps, P);
  if (blockIdx.x == 0 && tid == 0) a.ctl->splits = S;
  const int U = Tt * S;
  const int x = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int start = (int)(((int64_t)x * U) / 8), cnt = (int)(((int64_t)(x + 1) * U) / 8) - start;

  constexpr bool kPipe = use_pipe<T, D, NW, MET, KT, DHPART>();
  using PP = Pipe<D <= 128 ? D : 128, true, WITH_DH, kF16>;
  EN en;
  PP pp;
  if constexpr (kPipe) {
    pp.setup(lds, wave, lane);
    pp.X = (const char*)a.E;
    pp.x_bytes = a.V * (int64_t)D * 2;
    pp.Xsp = (const char*)a.Evp;
    pp.xsp_bytes = a.V_pad * (int64_t)D * 2;
    pp.bptr = a.bptr;
    pp.pairs = a.pairs;
  } else {
    en.setup(lds, wave, lane);
    en.X = (const T*)a.E;
    en.Xsp = (const T*)a.Evp;
    en.nX = a.V;
    en.bptr = a.bptr;
    en.pairs = a.pairs;
    en.apply_pos = a.pos_apply;
  }

  for (int idx = slot; idx < cnt; idx += P / 8) {
    const int u = start + idx;
    const int s = u / Tt, t = u % Tt;
    const int uj0 = (int)(((int64_t)s * n_steps) / S);
    const int uj1 = (int)(((int64_t)(s + 1) * n_steps) / S);
    const int r_base = t * RW + wave * 32;
    if constexpr (kPipe) {
      pp.j0 = uj0;
      pp.j1 = uj1;
      pp.bbase = (int64_t)t * a.n_vs;
      pp.own0 = r_base;
    } else {
      en.j0 = uj0;
      en.j1 = uj1;
      en.bbase = (int64_t)t * a.n_vs;
      en.own0 = r_base;
    }

    typename EL::Op hop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      hop[ks] = load_op<T>(Hc + (int64_t)(r_base + lane % 32) * D + ks * EL::kK + (lane / 32) * EL::kEPL);
    f32x16 acc[WITH_DH ? NDBE : 1];
#pragma unroll
    for (int db = 0; db < (WITH_DH ? NDBE : 1); ++db) acc[db] = f32x16{};
    float e_acc = 0.f, posz = 0.f;
    int met[3] = {0, 0, 0};
    TopK<KT ? KT : 1> tk;
    if (KT) tk.init();

    int poly_form = 0;  // epilogue the wave took (written per row for the finish)
    if constexpr (kPipe && kF16) {
      // |z| <= ||H[r]|| ||E[v]|| <= kPolyBoundF (kPolyBoundShort) for every logit of this wave: the polynomial
      // epilogue (its short form) applies
      float n2 = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = (float)((const bf16x8*)hop)[ks][j];
          n2 += x * x;
        }
      n2 += __shfl_xor(n2, 32, 64);  // the two halves of the row
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) n2 = fmaxf(n2, __shfl_xor(n2, o, 64));
      const float bound = sqrtf(n2) * __uint_as_float(a.ctl->enorm_max);
      const int form = __builtin_amdgcn_readfirstlane(bound <= kPolyBoundShort ? 2 : (bound <= kPolyBoundF ? 1 : 0));
      poly_form = form;
      if (form == 2)
        pp.template run<2>((const bf16x8*)hop, acc, e_acc, posz);
      else if (form == 1)
        pp.template run<1>((const bf16x8*)hop, acc, e_acc, posz);
      else
        pp.template run<0>((const bf16x8*)hop, acc, e_acc, posz);
    } else if constexpr (kPipe) {
      pp.run((const bf16x8*)hop, acc, e_acc, posz);
    } else
      en.run(hop, acc, e_acc, posz, met, &tk);

    // unit results: per-row loss parts and the dH partial of this split
    const int64_t urow = (int64_t)u * RW + wave * 32;  // row of the unit-major partial buffers
    if constexpr (KT > 0) {
      // merge the lists of the two lanes holding the row (the other lane's list is read whole before any
      // insertion changes it), then one lane writes it
      float ov[KT];
      int oi[KT];
#pragma unroll
      for (int q = 0; q < KT; ++q) {
        ov[q] = __shfl_xor(tk.v[q], 32, 64);
        oi[q] = __shfl_xor(tk.id[q], 32, 64);
      }
#pragma unroll
      for (int q = 0; q < KT; ++q) tk.template insert<false>(ov[q], oi[q]);
      if (lane < 32) {
#pragma unroll
        for (int q = 0; q < KT; ++q) {
          a.topv[(urow + lane) * KT + q] = tk.v[q];
          a.topi[(urow + lane) * KT + q] = tk.id[q];
        }
      }
      continue;
    }
    if (DHPART != 2) {
      const float e_tot = e_acc + __shfl_xor(e_acc, 32, 64);
      const float p_tot = posz + __shfl_xor(posz, 32, 64);
      if (lane < 32) a.rowpart[urow + lane] = make_float2(e_tot, p_tot);
    }
    if constexpr (std::is_same<T, __bf16>::value && evp_is_f16(1, D)) {
      // every split of the row writes the same flag (the wave's choice depends on its rows and all of E only)
      if (lane < 32) a.rowform[r_base + lane] = poly_form > 0 ? 1 : 0;
    }
    if (MET) {
#pragma unroll
      for (int q = 0; q < 3; ++q) met[q] += __shfl_xor(met[q], 32, 64);
      if (lane < 32) a.metpart[urow + lane] = make_int4(met[0], met[1], met[2], 0);
    }
    if (WITH_DH) {
      const float unscale = kF16 ? ldexpf(1.f, -evp_shift_of(a.ctl)) : 1.f;
#pragma unroll
      for (int db = 0; db < NDBE; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          a.dhpart[(urow + acc_pos(i, lane / 32)) * D + (DB0 + db) * 32 + lane % 32] = acc[db][i] * unscale;
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
  int64_t V, n_rs, R_pad;
  int n_full;        // item tiles swept whole; the tiles after them are swept in two row halves
  float* tailpart;   // [split tile][half][IW][D] fp32 partial sums of the halved tiles
};

// ---------------------------------------------------------------------------------------------------------
// Backward dE sweep: workgroup = item tile (32 items per wave), sweeping all valid rows.
// ---------------------------------------------------------------------------------------------------------
// DEPART 0: one pass; 1 / 2: the first / second of two passes, each accumulating and writing half of dE's
// d-blocks (half the accumulator registers, for f32 D = 256).
template <typename T, int D, int NW, int DEPART = 0>
__global__ void __launch_bounds__(NW * 64) k_items(ItemsArgs a) {
  using EL = Elem<T>;
  constexpr int NDB = D / 32, NDBE = DEPART ? NDB / 2 : NDB, DB0 = DEPART == 2 ? NDB / 2 : 0;
  // bf16: the gradient GEMM takes f16 G tiles and the f16 rows, scaled by 2^s (the sums are unscaled at the end)
  constexpr bool kF16 = std::is_same<T, __bf16>::value && hrp_is_f16(1, D);
  using EN = Engine<T, D, NW, false, true, false, 0, DB0, NDBE, true, kF16>;
  constexpr int IW = NW * 32, KS = D / EL::kK;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
  const T* __restrict__ E = (const T*)a.E;

  // Workgroups below n_full sweep a whole tile. The last tiles (fewer than half a round of workgroups) are
  // swept in two row halves by two workgroups each, which shortens the final round; their partial sums are
  // added by k_items_tail.
  const int b = blockIdx.x;
  const int split = b >= a.n_full ? (b - a.n_full) / 2 : -1;  // index among the halved tiles
  const int part = b >= a.n_full ? (b - a.n_full) % 2 : 0;
  const int t = split < 0 ? b : a.n_full + split;
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
  f32x16 acc[NDBE];
#pragma unroll
  for (int db = 0; db < NDBE; ++db) acc[db] = f32x16{};

  // clamped to the padded rows, so that no workspace contents can make the sweep run past them
  const int n_valid = min(max(a.ctl->n_valid, 0), (int)a.R_pad);
  const int n_st = (n_valid + 31) / 32;
  constexpr bool kPipe = use_pipe<T, D, NW, false, 0, DEPART>();
  if (kPipe && n_st > 0) {
    static_assert(!kPipe || hrp_is_f16(1, D), "the interleaved dE sweep reads f16 slot-packed rows");
    Pipe<D <= 128 ? D : 128, false, true, true> pp;
    pp.setup(lds, wave, lane);
    pp.X = (const char*)a.Hc;
    pp.x_bytes = a.R_pad * (int64_t)D * 2;
    pp.Xsp = (const char*)a.Hrp;
    pp.xsp_bytes = a.R_pad * (int64_t)D * 2;
    pp.bptr = a.bptr;
    pp.pairs = a.pairs;
    pp.bbase = (int64_t)t * a.n_rs;
    pp.own0 = (int)v_own0;
    pp.j0 = split < 0 || part == 0 ? 0 : n_st / 2;
    pp.j1 = split < 0 || part == 1 ? n_st : n_st / 2;
    float e_acc = 0.f, posz = 0.f;
    // |z| <= ||H[r]|| ||E[v]|| <= 1 for every logit of this wave: the polynomial epilogue applies
    float n2 = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = (float)((const bf16x8*)eop)[ks][j];
        n2 += x * x;
      }
    n2 += __shfl_xor(n2, 32, 64);  // the two halves of the item's row
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) n2 = fmaxf(n2, __shfl_xor(n2, o, 64));
    const float bound = sqrtf(n2) * __uint_as_float(a.ctl->hnorm_max);
    if (__builtin_amdgcn_readfirstlane(bound <= kPolyBound ? 1 : 0))
      pp.template run<1>((const bf16x8*)eop, acc, e_acc, posz);
    else
      pp.template run<0>((const bf16x8*)eop, acc, e_acc, posz);
  } else if (n_st > 0) {
    EN en;
    en.setup(lds, wave, lane);
    en.X = (const T*)a.Hc;
    en.Xsp = (const T*)a.Hrp;
    en.nX = n_valid;
    en.bptr = a.bptr;
    en.pairs = a.pairs;
    en.bbase = (int64_t)t * a.n_rs;
    en.own0 = (int)v_own0;
    en.j0 = split < 0 || part == 0 ? 0 : n_st / 2;
    en.j1 = split < 0 || part == 1 ? n_st : n_st / 2;
    float e_acc = 0.f, posz = 0.f;
    en.run(eop, acc, e_acc, posz, nullptr);
  }
  if (split >= 0) {
    float* __restrict__ tp = a.tailpart + ((int64_t)(split * 2 + part) * IW + wave * 32) * D;
#pragma unroll
    for (int db = 0; db < NDBE; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) tp[acc_pos(i, lane / 32) * D + (DB0 + db) * 32 + lane % 32] = acc[db][i];
    return;
  }

  // dE[v][d] = s * g * (acc + 1/2 sum_r H[r][d]); the f16 gradient GEMM summed rows scaled by 2^shift
  const double sc = a.ctl->scale * (double)a.grad_loss[0];
  const float scf = (float)sc;
  const float unscale = kF16 ? ldexpf(1.f, -hrp_shift(a.ctl->hw_absmax)) : 1.f;
  T* __restrict__ dE = (T*)a.dE;
#pragma unroll
  for (int db = 0; db < NDBE; ++db) {
    const int d = (DB0 + db) * 32 + lane % 32;
    const float half = (float)(0.5 * a.sumH[d]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t v = v_own0 + acc_pos(i, lane / 32);
      if (v < a.V) dE[v * D + d] = (T)(scf * (acc[db][i] * unscale + half));
    }
  }
}

// dE of the halved tiles: the two partial sums added in a fixed order, then scaled as in k_items. Grid:
// (halved tile, chunk of 1024 consecutive values); each thread handles 4 consecutive d of one item.
template <typename T, int IW, int D>
__global__ void __launch_bounds__(256) k_items_tail(ItemsArgs a) {
  static_assert(D % 4 == 0 && (IW * D) % 1024 == 0, "tail chunking");
  const int split = blockIdx.y;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;  // first value of this thread within the tile
  const int64_t v = (int64_t)(a.n_full + split) * IW + e / D;
  if (v >= a.V) return;
  const int d = e % D;
  const float scf = (float)(a.ctl->scale * (double)a.grad_loss[0]);
  const float4 p0 = *(const float4*)(a.tailpart + (int64_t)(split * 2) * IW * D + e);
  const float4 p1 = *(const float4*)(a.tailpart + (int64_t)(split * 2 + 1) * IW * D + e);
  // partial sums of the f16 gradient GEMM (bf16 inputs) are in units of 2^-shift
  const float us = std::is_same<T, __bf16>::value && hrp_is_f16(1, D) ? ldexpf(1.f, -hrp_shift(a.ctl->hw_absmax))
                                                                         : 1.f;
  const float q[4] = {(p0.x + p1.x) * us, (p0.y + p1.y) * us, (p0.z + p1.z) * us, (p0.w + p1.w) * us};
  T* __restrict__ out = (T*)a.dE + v * D + d;
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = (T)(scf * (q[k] + (float)(0.5 * a.sumH[d + k])));
}

// ---------------------------------------------------------------------------------------------------------
// The 16-owner engine (bf16, D = 256 and 512). A wave owns 16 rows (forward) or 16 items (dE) and streams 32
// per step through the rings of Engine, on 16x16x32 MFMA tiles: the owner operand (D / 32 registers of 8 values)
// and the gradient accumulators (D / 16 tiles of 4 registers) fit two waves per SIMD even at D = 512, where a
// 32-owner wave needs twice as many and runs alone on its SIMD (the forward then in two passes). Each MFMA takes
// one 16-byte LDS read, as the 32x32x16 engines do for twice the work; the epilogue has 8 values per lane and
// step against 2 * D / 16 MFMAs.
//
// Logit tile of step j, half h (streamed 16h..16h+15): A = streamed rows from the d-packed block, B = owner
// operand, so lane l holds z[h][i] of owner l % 16 and streamed 16h + 4(l/16) + i. Its 8 values, in the order
// 4h + i, are the lane's k-slots 8(l/16) .. 8(l/16) + 7 of the gradient GEMM: A = G (owner l % 16), B = the
// slot-packed block (sp16_row gives each slot's streamed row), acc[db] holds owner 4(l/16) + i, d = 16 db + l % 16.
// ---------------------------------------------------------------------------------------------------------

// Forward epilogue on 8 logits of one lane (the 16-value form of epi_rows with one quad pair fewer).
template <bool GRAD, bool LOSS>
__device__ inline void epi_rows8(const float* z, float* c, float& e_acc) {
  float w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = 1.f + __builtin_amdgcn_exp2f(z[i] * -kLog2e);
  float w2[4], w4[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) w2[i] = w[2 * i] * w[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 2; ++i) w4[i] = w2[2 * i] * w2[2 * i + 1];
  const float wp = w4[0] * w4[1];
  if (GRAD) inv_minus_half<2>(w, w2, w4, c);
  float e_inc = LOSS ? kLn2 * (__builtin_amdgcn_logf(wp) - 8.f) : 0.f;
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(wp <= kFastProd)) != 0, 0)) {
    float u[8], wa[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u[i] = __builtin_fabsf(z[i]) * -kLog2e;
      wa[i] = 1.f + __builtin_amdgcn_exp2f(u[i]);
    }
    float a2[4], a4[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) a2[i] = wa[2 * i] * wa[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 2; ++i) a4[i] = a2[2 * i] * a2[2 * i + 1];
    if (GRAD) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float r4 = __builtin_amdgcn_rcpf(a4[q]);
        const float ra = r4 * a2[2 * q + 1], rb = r4 * a2[2 * q];
        const float r[4] = {ra * wa[4 * q + 1], ra * wa[4 * q], rb * wa[4 * q + 3], rb * wa[4 * q + 2]};
#pragma unroll
        for (int k = 0; k < 4; ++k) c[4 * q + k] = __builtin_copysignf(r[k] - 0.5f, z[4 * q + k]);
      }
    }
    if (LOSS) {
      float us = 0.f, zs = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        us += u[i];
        zs += z[i];
      }
      e_inc = kLn2 * (__builtin_amdgcn_logf(a4[0] * a4[1]) - 8.f - 0.5f * us) - 0.5f * zs;
    }
  }
  if (LOSS) e_acc += e_inc;
}

// dE epilogue on 8 logits: c = 1/(1 + e^-z) - 1/2.
__device__ inline void epi_items8(const float* z, float* c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(z[i] * -kLog2e)) - 0.5f;
}

// Per-lane positive mask of a 16-owner step: bit 4h + i of lane o + 16 q is the pair (owner o, streamed
// 16h + 4q + i). Same bucket walk as positive_mask.
__device__ inline uint32_t positive_mask16(const int2* __restrict__ pairs, int pb, int pe, int own, int stream0,
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
      if (o >= 0 && o < 16 && sidx >= 0 && sidx < 32)
        atomicOr(&lmask[o + 16 * ((sidx >> 2) & 3)], 1u << (4 * (sidx >> 4) + (sidx & 3)));
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  return lmask[lane];
}

// The 8-value epilogues of epi_rows8 / epi_items8 cut into stages, so that the 16-owner engine can place them
// between the MFMAs of an iteration (same operations, same order of rounding; the forward's |z| form runs in
// finish(), after the MFMAs, and only when a lane's product passes kFastProd).
template <bool FWD, bool GRAD>
struct Epi8 {
  static constexpr int NS = FWD ? (GRAD ? 6 : 4) : 5;  // stages
  float z[8], t[8], c[8], w2[4], w4[2], r4[2], lg;
  __device__ inline void stage(int st) {
    if (st == 0 || st == 1) {
#pragma unroll
      for (int i = 4 * st; i < 4 * st + 4; ++i)
        t[i] = FWD ? 1.f + __builtin_amdgcn_exp2f(z[i] * -kLog2e) : __builtin_amdgcn_exp2f(z[i] * -kLog2e);
      return;
    }
    if constexpr (FWD) {
      if (st == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w2[i] = t[2 * i] * t[2 * i + 1];
        w4[0] = w2[0] * w2[1];
        w4[1] = w2[2] * w2[3];
      } else if (st == 3) {
        lg = __builtin_amdgcn_logf(w4[0] * w4[1]);
        if (GRAD) {
          r4[0] = __builtin_amdgcn_rcpf(w4[0]);
          r4[1] = __builtin_amdgcn_rcpf(w4[1]);
        }
      } else if (GRAD && (st == 4 || st == 5)) {
        const int q = st - 4;  // inv_minus_half for quad q
        const float ra = r4[q] * w2[2 * q + 1], rb = r4[q] * w2[2 * q];
        c[4 * q] = ra * t[4 * q + 1] - 0.5f;
        c[4 * q + 1] = ra * t[4 * q] - 0.5f;
        c[4 * q + 2] = rb * t[4 * q + 3] - 0.5f;
        c[4 * q + 3] = rb * t[4 * q + 2] - 0.5f;
      }
    } else {
      if (st == 2) {
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = 1.f + t[i];
      } else if (st == 3 || st == 4) {
#pragma unroll
        for (int i = 4 * (st - 3); i < 4 * (st - 3) + 4; ++i) c[i] = __builtin_amdgcn_rcpf(t[i]) - 0.5f;
      }
    }
  }
  // Runs the stages in one go (an iteration that deals none out).
  __device__ inline void all_stages() {
#pragma unroll
    for (int st = 0; st < NS; ++st) stage(st);
  }
  // forward: the loss term (or the |z| form of loss and c for a tile whose product passes kFastProd)
  __device__ inline void finish(float& e_acc) {
    if constexpr (FWD) {
      const float wp = w4[0] * w4[1];
      float e_inc = kLn2 * (lg - 8.f);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(wp <= kFastProd)) != 0, 0)) {
        float u[8], wa[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          u[i] = __builtin_fabsf(z[i]) * -kLog2e;
          wa[i] = 1.f + __builtin_amdgcn_exp2f(u[i]);
        }
        float a2[4], a4[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) a2[i] = wa[2 * i] * wa[2 * i + 1];
#pragma unroll
        for (int i = 0; i < 2; ++i) a4[i] = a2[2 * i] * a2[2 * i + 1];
        if (GRAD) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float rr = __builtin_amdgcn_rcpf(a4[q]);
            const float ra = rr * a2[2 * q + 1], rb = rr * a2[2 * q];
            const float x[4] = {ra * wa[4 * q + 1], ra * wa[4 * q], rb * wa[4 * q + 3], rb * wa[4 * q + 2]};
#pragma unroll
            for (int k = 0; k < 4; ++k) c[4 * q + k] = __builtin_copysignf(x[k] - 0.5f, z[4 * q + k]);
          }
        }
        float us = 0.f, zs = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          us += u[i];
          zs += z[i];
        }
        e_inc = kLn2 * (__builtin_amdgcn_logf(a4[0] * a4[1]) - 8.f - 0.5f * us) - 0.5f * zs;
      }
      e_acc += e_inc;
    }
  }
};

// PAIR (forward, D = 512): waves 2p and 2p + 1 own the same 16 rows and split the features: wave 2p + s holds
// the owner operand and the dH accumulators of d in [s D/2, (s + 1) D/2), so each forms a partial logit tile over
// its half. The partials go through LDS (two slots per wave, written in iteration i for step i + 1 and read after
// the barrier of iteration i + 1) and both waves add them in the same order (half 0's + half 1's), so both hold
// the same logits and G tile. 96 registers per wave instead of 192 give two waves per SIMD without spilling, and
// no MFMA is repeated; the epilogue is computed by both waves.
template <int D, bool FWD, bool GRAD, bool MET, int NW = 8, bool PAIR = false,
          bool POS = !FWD || MET || !kGatherPositives>
struct Eng16 {
  static constexpr int KB = D / 32, NDB = D / 16;
  static constexpr int KBW = PAIR ? KB / 2 : KB, NDBW = PAIR ? NDB / 2 : NDB;  // this wave's k- and d-blocks
  static_assert(!PAIR || (FWD && !POS && NW == 8), "paired waves: the forward without positives");
  // One wave per SIMD (NW = 4): the epilogue's stages are dealt out between the MFMAs and the whole order is
  // pinned, since no other wave fills the vector ALU; two waves per SIMD (NW = 8): the compiler places the
  // vector work between the pinned MFMAs and LDS reads.
  static constexpr bool kStaged = NW == 4;
  using R = Engine<__bf16, D, NW, FWD, GRAD, MET>;  // rings, their loads and barriers, bucket pointers
  using G = Geo<__bf16, D, NW, GRAD>;
  using GOp = typename std::conditional<FWD, bf16x8, f16x8>::type;  // dE: f16 G and f16 slot-packed rows
  struct Z {
    f32x4 h[2];
  };
  R r;
  bool apply_pos = true;
  int half = 0;        // PAIR: this wave's feature half
  uint32_t xoff = 0;   // PAIR: LDS byte offset of the partial-logit exchange (2 slots x NW waves x 2 KB)
  static constexpr int kXchgBytes = PAIR ? 2 * NW * 64 * 32 : 0;
  __device__ inline void setup(char* l, int w, int ln) {
    r.setup(l, w, ln);
    half = PAIR ? r.wave % 2 : 0;
    xoff = (G::kNA + G::kNB) * G::kStepBytes;
  }
  static constexpr size_t lds_bytes() {
    return PAIR ? (size_t)(G::kNA + G::kNB) * G::kStepBytes + kXchgBytes : (size_t)G::kLdsBytes;
  }
  // PAIR: this wave's partial logits of a step into exchange slot `slot`; the full tile from the two partials
  __device__ inline void put_partial(int slot, const Z& z) const {
    f32x4* x = (f32x4*)(r.lds + xoff + ((slot * NW + r.wave) * 64 + r.lane) * 32);
    x[0] = z.h[0];
    x[1] = z.h[1];
  }
  __device__ inline void full_logits(int slot, const Z& mine, float* zf) const {
    const f32x4* x = (const f32x4*)(r.lds + xoff + ((slot * NW + (r.wave ^ 1)) * 64 + r.lane) * 32);
    const f32x4 o0 = x[0], o1 = x[1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      zf[q] = half == 0 ? mine.h[0][q] + o0[q] : o0[q] + mine.h[0][q];
      zf[4 + q] = half == 0 ? mine.h[1][q] + o1[q] : o1[q] + mine.h[1][q];
    }
  }

  // The A ring holds each step's block operand-major: the 1 KB at (2 kb + h) * 1024 is the A operand of k-block
  // kb, half h, lane l's 16 bytes at l * 16 (streamed row 16h + l%16, features 32 kb + 8 (l/16) .. + 7). The DMA
  // writes 16 bytes per lane at consecutive LDS addresses from a per-lane global offset, so the permutation costs
  // nothing there, and every operand read is conflict-free at one lane address plus a constant.
  __device__ inline void dma_a(int rel, int slot) const {
    const int64_t row0 = (int64_t)r.clampj(rel) * 32;
    const char* xa = (const char*)r.X + row0 * (int64_t)(D * 2);
    const int64_t rem = (r.nX - row0) * (int64_t)(D * 2);
    const int nrec = rem <= 0 ? 0 : (rem > (int64_t)G::kStepBytes ? G::kStepBytes : (int)rem);
    __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)xa, (short)0, nrec, 0x00020000);
    const uint32_t dst = r.lds_s + slot * G::kStepBytes;
    static_assert(G::kLoadB == 16 && G::kWaveBytes == 1024, "one 1 KB operand per wave instruction");
#pragma unroll
    for (int q = 0; q < G::kLoadsPerPart; ++q) {
      const int inst = r.wave + q * NW;  // operand (kb, h) = (inst / 2, inst % 2)
      const int voff = (16 * (inst % 2) + r.lane % 16) * (D * 2) + (32 * (inst / 2) + 8 * (r.lane / 16)) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(size_t)(dst + inst * 1024), 16, voff, 0, 0, 0);
    }
  }
  // Start of iteration i: the barrier (every kK iterations, with the bucket refill) and the iteration's loads.
  __device__ inline void top(int i) {
    if (G::kK == 1 || i % G::kK == 0) {
      if (POS)
        r.barrier_at(i);
      else
        wait_vm_and_barrier<G::kInFlight>();
    }
    dma_a(i + G::kLA, (i + G::kLA) % G::kNA);
    if (GRAD) r.dma_b(i + G::kLB);
  }
  using EP = Epi8<FWD, GRAD>;
  // End of step j's epilogue, after its stages: loss, positives of the step (bucket [pb, pe)), Cut Metrics counts,
  // the G tile.
  __device__ inline void epilogue_end(int j, int pb, int pe, EP& es, GOp& g, float& posz, int* met) {
    uint32_t gt = 0u;  // bit q: z[q] > 0 (Cut Metrics)
    if (MET) {
#pragma unroll
      for (int q = 0; q < 8; ++q) gt |= (es.z[q] > 0.f ? 1u : 0u) << q;
      met[0] += __builtin_popcount(gt);
    }
    if (POS && pe > pb) {
      const uint32_t pm = positive_mask16(r.pairs, pb, pe, r.own0, (r.j0 + j) * 32, FWD, r.lmask(), r.lane);
      if (pm) {
        if (apply_pos) {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (pm & (1u << q)) {
              if (FWD) posz += es.z[q];
              if (GRAD) es.c[q] -= 1.f;
            }
        }
        if (MET) {
          met[1] += __builtin_popcount(pm & gt);
          met[2] += __builtin_popcount(pm);
        }
      }
    }
    if (GRAD) {
#pragma unroll
      for (int q = 0; q < 8; ++q) g[q] = (typename std::conditional<FWD, __bf16, _Float16>::type)es.c[q];
    }
  }
  // Iteration i: ring loads and barrier, logits of step i + 1 (into zn; NEXT), gradient GEMM of step i - 1 (PREV),
  // epilogue of step i (zc). MFMA order: per k-block, logit half 0, gradient d-block 2kb, logit half 1, gradient
  // d-block 2kb + 1 (a logit chain's MFMAs four apart). Each MFMA's LDS operand is read three MFMAs ahead into a
  // ring of four registers, and the epilogue's stages are dealt out between the MFMAs; the whole order is pinned
  // (sched_barrier): the compiler would otherwise either hoist every read of the iteration or, short of
  // registers, wait for each read right before its MFMA, and it left the forward's epilogue after the MFMAs. The
  // first and last iterations are peeled, so the main loop has no conditions.
  // The pinned MFMA sequence: logits into zn from the A slot of step ia (kL), gradient GEMM into acc from the B
  // slot of step ig (kG).
  template <bool kL, bool kG, bool kE = false>
  __device__ inline void mfma_seq(int ia, int ig, const bf16x8* own, Z& zn, const GOp& g, f32x4* acc,
                                  EP* es = nullptr) const {
    constexpr int NM = (kL ? 2 * KBW : 0) + (kG ? NDBW : 0);
    constexpr int PER = kE ? (NM / EP::NS > 0 ? NM / EP::NS : 1) : 1;  // MFMAs per epilogue stage
    const char* pa = r.lds + (ia % G::kNA) * G::kStepBytes + r.lane * 16 + half * (KBW * 2 * 1024);
    const char* pg = r.lds + (G::kNA + ig % (G::kNB ? G::kNB : 1)) * G::kStepBytes + r.lane * 16 + half * (NDBW * 1024);
    // The one-wave D = 512 forward (Cut Metrics) sums its logits over the two feature halves separately and adds
    // the halves, as the paired waves do, so that both forms give the same bits.
    constexpr bool kHalves = FWD && D == 512 && !PAIR;
    Z zx;  // kHalves: the second feature half
    if (kL) {
      zn.h[0] = f32x4{};
      zn.h[1] = f32x4{};
      if (kHalves) zx = zn;
    }
    // MFMA k: logit (k-block, half) or gradient (d-block)
    auto is_l = [](int k) { return kL && (!kG || (k & 1) == 0); };
    auto l_kb = [](int k) { return kG ? k / 4 : k / 2; };
    auto l_h = [](int k) { return kG ? (k / 2) & 1 : k & 1; };
    auto g_db = [](int k) { return kL ? 2 * (k / 4) + ((k / 2) & 1) : k; };
    auto read = [&](int k) -> u32x4 {
      return is_l(k) ? *(const u32x4*)(pa + (2 * l_kb(k) + l_h(k)) * 1024) : *(const u32x4*)(pg + g_db(k) * 1024);
    };
    // operand ring, reads RB - 1 MFMAs ahead; measured: 6 for the D = 256 forward (-6.5% at 4,096 rows x 10M
    // items), no gain for the dE sweeps or the paired D = 512 forward
    constexpr int RB = (NW == 4 || (FWD && D == 256)) ? 6 : 4;
    u32x4 buf[RB];
#pragma unroll
    for (int k = 0; k < RB - 1; ++k)
      if (k < NM) buf[k] = read(k);
#pragma unroll
    for (int k = 0; k < NM; ++k) {
      if (k + RB - 1 < NM) buf[(k + RB - 1) % RB] = read(k + RB - 1);
      const u32x4 op = buf[k % RB];
      if (is_l(k)) {
        const int h = l_h(k);
        if (kHalves && l_kb(k) >= KB / 2)
          zx.h[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, op), own[l_kb(k)], zx.h[h],
                                                            0, 0, 0);
        else
          zn.h[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, op), own[l_kb(k)], zn.h[h],
                                                            0, 0, 0);
      } else if constexpr (FWD) {
        acc[g_db(k)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g, __builtin_bit_cast(bf16x8, op), acc[g_db(k)], 0, 0,
                                                               0);
      } else {
        acc[g_db(k)] = __builtin_amdgcn_mfma_f32_16x16x32_f16(g, __builtin_bit_cast(f16x8, op), acc[g_db(k)], 0, 0,
                                                              0);
      }
      if (kE && k % PER == PER - 1 && k / PER < EP::NS) es->stage(k / PER);
      __builtin_amdgcn_sched_barrier(kStaged ? 0 : 0x0406);  // unstaged: VALU, SALU, transcendentals may cross
    }
    if (kE && NM / PER < EP::NS) {  // stages left over (a sequence shorter than the epilogue)
#pragma unroll
      for (int st = NM / PER; st < EP::NS; ++st) es->stage(st);
    }
    if (kHalves && kL) {
      zn.h[0] = zn.h[0] + zx.h[0];
      zn.h[1] = zn.h[1] + zx.h[1];
    }
  }
  template <bool NEXT, bool PREV>
  __device__ inline void iter(int i, const bf16x8* own, const Z& zc, Z& zn, GOp& g, f32x4* acc, float& e_acc,
                              float& posz, int* met) {
    __builtin_amdgcn_sched_barrier(0);
    top(i);
    int pb = 0, pe = 0;
    if (POS) r.bkt_get(i, pb, pe);
    EP es;
    if (PAIR) {
      full_logits(i % 2, zc, es.z);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) es.z[q] = zc.h[q / 4][q % 4];
    }
    if (kStaged) {
      mfma_seq<NEXT, GRAD && PREV, true>(i + 1, i - 1, own, zn, g, acc, &es);
    } else {
      mfma_seq<NEXT, GRAD && PREV, false>(i + 1, i - 1, own, zn, g, acc);
      es.all_stages();
    }
    if (PAIR && NEXT) put_partial((i + 1) % 2, zn);
    es.finish(e_acc);
    epilogue_end(i, pb, pe, es, g, posz, met);
  }
  __device__ inline void run(const bf16x8* own, f32x4* acc, float& e_acc, float& posz, int* met) {
    const int n = r.j1 - r.j0;
    if (n <= 0) return;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // everyone is done with the previous unit's rings
#pragma unroll
    for (int q = 0; q < G::kLA; ++q) dma_a(q, q % G::kNA);
    if (GRAD) {
#pragma unroll
      for (int q = 0; q < G::kLB; ++q) r.dma_b(q);
    }
    if (POS) r.bkt_init();
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    static_assert(!PAIR || G::kK == 1, "paired waves exchange partial logits across the barrier of every step");
    GOp g;
    Z zc, zn;
    mfma_seq<true, false>(0, 0, own, zc, g, acc);  // step 0
    if (PAIR) put_partial(0, zc);
    if (n == 1) {
      iter<false, false>(0, own, zc, zn, g, acc, e_acc, posz, met);
    } else {
      iter<true, false>(0, own, zc, zn, g, acc, e_acc, posz, met);
      for (int i = 1; i < n - 1; ++i) {
        zc = zn;  // eight moves per 2 * D / 16 MFMAs
        iter<true, true>(i, own, zc, zn, g, acc, e_acc, posz, met);
      }
      zc = zn;
      iter<false, true>(n - 1, own, zc, zn, g, acc, e_acc, posz, met);
    }
    wait_vm_and_barrier<0>();  // the slot-packed block of step n - 1 has landed
    if (GRAD) mfma_seq<false, true>(0, n - 1, own, zn, g, acc);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
};

// Forward sweep on the 16-owner engine: the unit loop, splits and partial layouts of k_rows (row tiles of NW waves
// x 16 rows: 128 at D = 256, two waves per SIMD; 64 at D = 512, one wave per SIMD).
template <int D, bool WITH_DH, bool MET, int NW, bool PAIR>
__global__ void __launch_bounds__(NW * 64) k_rows16(RowsArgs a) {
  using EN = Eng16<D, true, WITH_DH, MET, NW, PAIR>;
  constexpr int RW = (PAIR ? NW / 2 : NW) * 16, KB = EN::KBW, NDB = EN::NDBW;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
  const __bf16* __restrict__ Hc = (const __bf16*)a.Hc;
  const int n_valid = a.ctl->n_valid;
  const int Tt = (n_valid + RW - 1) / RW;
  if (Tt == 0) return;
  const int n_steps = (int)(a.V_pad / 32);
  const int P = gridDim.x;
  const int S = choose_splits(Tt, n_steps, P);
  if (blockIdx.x == 0 && tid == 0) a.ctl->splits = S;
  const int U = Tt * S;
  const int x = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int start = (int)(((int64_t)x * U) / 8), cnt = (int)(((int64_t)(x + 1) * U) / 8) - start;
  EN en;
  en.setup(lds, wave, lane);
  en.r.X = (const __bf16*)a.E;
  en.r.Xsp = (const __bf16*)a.Evp;
  en.r.nX = a.V;
  en.r.bptr = a.bptr;
  en.r.pairs = a.pairs;
  en.apply_pos = a.pos_apply;
  for (int idx = slot; idx < cnt; idx += P / 8) {
    const int u = start + idx;
    const int s = u / Tt, t = u % Tt;
    const int wrow = PAIR ? wave / 2 : wave;  // the wave's 16 rows within the tile
    const int r_base = t * RW + wrow * 16;
    en.r.j0 = (int)(((int64_t)s * n_steps) / S);
    en.r.j1 = (int)(((int64_t)(s + 1) * n_steps) / S);
    en.r.bbase = (int64_t)t * a.n_vs;
    en.r.own0 = r_base;
    // lane addresses made opaque, so that the compiler does not hoist per-offset partial addresses out of the
    // unit loop (they would stay live across it)
    const __bf16* hp = Hc + (int64_t)(r_base + lane % 16) * D + en.half * (D / 2) + (lane / 16) * 8;
    asm volatile("" : "+v"(hp));
    bf16x8 hop[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) hop[kb] = *(const bf16x8*)(hp + kb * 32);
    f32x4 acc[WITH_DH ? NDB : 1];
#pragma unroll
    for (int db = 0; db < (WITH_DH ? NDB : 1); ++db) acc[db] = f32x4{};
    float e_acc = 0.f, posz = 0.f;
    int met[3] = {0, 0, 0};
    en.run(hop, acc, e_acc, posz, met);
    // lanes o, o + 16, o + 32, o + 48 hold row o's sums
    const int64_t urow = (int64_t)u * RW + wrow * 16;
    float e_tot = e_acc + __shfl_xor(e_acc, 16, 64), p_tot = posz + __shfl_xor(posz, 16, 64);
    e_tot += __shfl_xor(e_tot, 32, 64);
    p_tot += __shfl_xor(p_tot, 32, 64);
    if (lane < 16 && en.half == 0) a.rowpart[urow + lane] = make_float2(e_tot, p_tot);
    if (MET) {
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        met[q] += __shfl_xor(met[q], 16, 64);
        met[q] += __shfl_xor(met[q], 32, 64);
      }
      if (lane < 16) a.metpart[urow + lane] = make_int4(met[0], met[1], met[2], 0);
    }
    if (WITH_DH) {
      float* dp = a.dhpart + (urow + 4 * (lane / 16)) * D + en.half * (D / 2) + lane % 16;
      asm volatile("" : "+v"(dp));
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) dp[i * D + db * 16] = acc[db][i];
    }
  }
}

// dE sweep on the 16-owner engine: item tiles of 8 waves x 16 items = 128, halved tail tiles as in k_items.
template <int D>
__global__ void __launch_bounds__(512) k_items16(ItemsArgs a) {
  using EN = Eng16<D, false, true, false>;
  constexpr int IW = 128, KB = D / 32, NDB = D / 16;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
  const __bf16* __restrict__ E = (const __bf16*)a.E;
  const int b = blockIdx.x;
  const int split = b >= a.n_full ? (b - a.n_full) / 2 : -1;
  const int part = b >= a.n_full ? (b - a.n_full) % 2 : 0;
  const int t = split < 0 ? b : a.n_full + split;
  const int64_t v_own0 = (int64_t)t * IW + wave * 16;  // first item of this wave
  const int64_t v_mine = v_own0 + lane % 16;
  bf16x8 eop[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    eop[kb] = v_mine < a.V ? *(const bf16x8*)(E + v_mine * D + kb * 32 + (lane / 16) * 8) : bf16x8{};
  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{};
  const int n_valid = min(max(a.ctl->n_valid, 0), (int)a.R_pad);
  const int n_st = (n_valid + 31) / 32;
  if (n_st > 0) {
    EN en;
    en.setup(lds, wave, lane);
    en.r.X = (const __bf16*)a.Hc;
    en.r.Xsp = (const __bf16*)a.Hrp;  // f16 values; the ring copies bytes
    en.r.nX = n_valid;
    en.r.bptr = a.bptr;
    en.r.pairs = a.pairs;
    en.r.bbase = (int64_t)t * a.n_rs;
    en.r.own0 = (int)v_own0;
    en.r.j0 = split < 0 || part == 0 ? 0 : n_st / 2;
    en.r.j1 = split < 0 || part == 1 ? n_st : n_st / 2;
    float e_acc = 0.f, posz = 0.f;
    en.run(eop, acc, e_acc, posz, nullptr);
  }
  if (split >= 0) {
    float* __restrict__ tp = a.tailpart + ((int64_t)(split * 2 + part) * IW + wave * 16) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) tp[(4 * (lane / 16) + i) * D + db * 16 + lane % 16] = acc[db][i];
    return;
  }
  // dE[v][d] = s * g * (acc * 2^-shift + 1/2 sum_r w_r H[r][d])
  const float scf = (float)(a.ctl->scale * (double)a.grad_loss[0]);
  const float unscale = ldexpf(1.f, -hrp_shift(a.ctl->hw_absmax));
  __bf16* __restrict__ dE = (__bf16*)a.dE;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d = db * 16 + lane % 16;
    const float half = (float)(0.5 * a.sumH[d]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t v = v_own0 + 4 * (lane / 16) + i;
      if (v < a.V) dE[v * D + d] = (__bf16)(scf * (acc[db][i] * unscale + half));
    }
  }
}

// ---------------------------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------------------------
constexpr int kMaxDevices = 16;  // devices whose launch data is cached (others query every time)

// Compute units of the current device, cached per device.
static int cu_count() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const int slot = dev >= 0 && dev < kMaxDevices ? dev : -1;
  int n = slot >= 0 ? cached[slot].load(std::memory_order_relaxed) : 0;
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (slot >= 0) cached[slot].store(n, std::memory_order_relaxed);
  return n;
}

// Once per kernel and device: the dynamic-LDS limit and the number of workgroups resident per CU (both fixed
// for a kernel). Later launches then make no runtime call but the launch itself, which also keeps them
// capturable into a graph.
template <auto Kern>
static hipError_t kernel_setup(int threads, size_t sm, int& per_cu) {
  static std::atomic<int> cached[kMaxDevices];  // resident workgroups per CU; 0 = not set up yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  if (dev >= 0 && (per_cu = cached[dev].load(std::memory_order_relaxed)) > 0) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)Kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)Kern, threads, sm) != hipSuccess || n < 1) n = 1;
  per_cu = n;
  if (dev >= 0) cached[dev].store(n, std::memory_order_relaxed);
  return hipSuccess;
}

// Gradient accumulators (NDB tiles of 16 registers) plus the owner operand (D / k-per-MFMA operands) per lane:
// when they fill the 256 registers of a wave, the 32-owner sweeps can run as two passes over half of the
// gradient's d-blocks each, recomputing the logits instead of spilling: used for f32 D = 256 (forward 26.4 ->
// 17.2 ms at 4,096 rows x 131,072 items); bf16 D = 256 and 512 run the 16-owner engine instead.
template <typename T, int D>
constexpr bool two_pass() {
  return (D / 32) * 16 + (D / Elem<T>::kK) * (int)(sizeof(typename Elem<T>::Op) / 4) >= 256;
}

// Item tiles of the dE sweep swept by two workgroups over the two halves of the rows (k_items_tail adds the
// halves): the tiles of the last round when it would be at most half full, or every tile when all of them fill at
// most half of the P resident workgroups (at 6,400 rows x 100,000 items, 391 tiles of 256 items for 768 slots)
// and the partial-sum area holds them (cap halved tiles).
static int64_t halved_tiles(int64_t n_vt, int64_t P, int64_t rem, int64_t cap) {
  if (n_vt > P) return (rem > 0 && 2 * rem <= P) ? rem : 0;
  return 2 * n_vt <= P && n_vt <= cap ? n_vt : 0;
}

// Forward-sweep grid: persistent, as many workgroups as can be resident at once (per_cu per CU), a multiple of
// 8 (one range per XCD). The kernel derives its vocabulary splits from the grid size.
static int persistent_grid(int per_cu) {
  const int P = (cu_count() * per_cu / 8) * 8;
  return P > 0 ? P : 8;
}

static RowsArgs rows_args(const Layout& L, char* ws, const void* E, bool pos_apply, int KT) {
  RowsArgs a;
  a.pos_apply = pos_apply;
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
  a.rowform = (uint8_t*)(ws + L.off_rowform);
  a.rowpart = (float2*)(ws + L.off_rowpart);
  a.metpart = (int4*)(ws + L.off_metpart);
  a.topv = (float*)(ws + L.off_dhpart);
  a.topi = (int32_t*)(ws + L.off_dhpart) + (size_t)L.part_rows * (KT ? KT : 1);
  return a;
}

// Forward sweep of bf16 D = 256 / 512 on the 16-owner engine (one pass; the same row tiles of 128 and partials).
template <int D, bool WITH_DH, bool MET>
static hipError_t rows_launch16(const Layout& L, char* ws, const void* E, hipStream_t st, bool pos_apply) {
  // D = 512: paired waves (two per SIMD), or with Cut Metrics (which needs the positives' mask area) one wave
  // per SIMD over whole rows; both keep 64-row tiles
  constexpr bool PAIR = D == 512 && !MET && !(!kGatherPositives);
  constexpr int NW = PAIR ? 8 : rows16_waves(D);
  if (L.rows_per_wg != (PAIR ? NW / 2 : NW) * 16) return hipErrorInvalidValue;  // the layout's row tiles
  const RowsArgs a = rows_args(L, ws, E, pos_apply, 0);
  constexpr auto kern = k_rows16<D, WITH_DH, MET, NW, PAIR>;
  const size_t sm = Eng16<D, true, WITH_DH, MET, NW, PAIR>::lds_bytes();
  int per_cu = 1;
  hipError_t e = kernel_setup<kern>(NW * 64, sm, per_cu);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(persistent_grid(per_cu)), dim3(NW * 64), sm, st, a);
  return hipGetLastError();
}

template <typename T, int D, int NW, bool WITH_DH, bool MET, int KT = 0>
static hipError_t rows_launch(const Layout& L, char* ws, const void* E, hipStream_t st, bool pos_apply = true) {
  if constexpr (KT == 0 && narrow_owner(sizeof(T) == 2 ? 1 : 0, D)) {
    static_assert(NW * 32 == rows16_waves(D) * 16, "the scoring engine and the 16-owner engine share row tiles");
    return rows_launch16<D, WITH_DH, MET>(L, ws, E, st, pos_apply);
  } else {
    // scoring partials reuse the dH partial area: KT * 8 bytes per row <= D * 4 bytes
    static_assert(KT * 8 <= D * 4, "top-k partials fit in the dH partial area");
    const RowsArgs a = rows_args(L, ws, E, pos_apply, KT);
    // Both passes run on the same grid, hence the same vocabulary splits and partial-sum layout.
    constexpr bool kTwoPass = WITH_DH && KT == 0 && two_pass<T, D>();
    if constexpr (kTwoPass) {
      const size_t sm = Geo<T, D, NW, WITH_DH>::kLdsBytes;
      constexpr auto k1 = k_rows<T, D, NW, WITH_DH, MET, KT, 1>;
      constexpr auto k2 = k_rows<T, D, NW, WITH_DH, false, KT, 2>;
      int c1 = 1, c2 = 1;
      hipError_t e = kernel_setup<k1>(NW * 64, sm, c1);
      if (e != hipSuccess) return e;
      if ((e = kernel_setup<k2>(NW * 64, sm, c2)) != hipSuccess) return e;
      const int P = persistent_grid(c1 < c2 ? c1 : c2);
      hipLaunchKernelGGL(k1, dim3(P), dim3(NW * 64), sm, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL(k2, dim3(P), dim3(NW * 64), sm, st, a);
      return hipGetLastError();
    } else {
      constexpr auto kern = k_rows<T, D, NW, WITH_DH, MET, KT>;
      const size_t sm1 = sweep_lds<T, D, NW, true, WITH_DH, MET, KT, 0>();
      int per_cu = 1;
      hipError_t e = kernel_setup<kern>(NW * 64, sm1, per_cu);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, dim3(persistent_grid(per_cu)), dim3(NW * 64), sm1, st, a);
      return hipGetLastError();
    }
  }
}

// dE sweep of bf16 D = 256 / 512 on the 16-owner engine (item tiles of 128, halved tail tiles as in items_launch).
template <int D>
static hipError_t items_launch16(const Layout& L, char* ws, const void* E, const float* grad_loss, void* dE,
                                 hipStream_t st) {
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
  a.R_pad = L.R_pad;
  constexpr auto kern = k_items16<D>;
  const size_t sm = Geo<__bf16, D, 8, true>::kLdsBytes;
  int per_cu = 1;
  hipError_t e = kernel_setup<kern>(512, sm, per_cu);
  if (e != hipSuccess) return e;
  const int64_t P = (int64_t)cu_count() * per_cu;
  const int64_t rem = L.n_vt % P;
  const int64_t n_split = halved_tiles(L.n_vt, P, rem, L.part_rows / 256);
  a.n_full = (int)(L.n_vt - n_split);
  a.tailpart = (float*)(ws + L.off_dhpart);
  if (L.items_per_wg != 128 || n_split * 2 > L.part_rows / 128) return hipErrorInvalidValue;  // cannot happen
  hipLaunchKernelGGL(kern, dim3((unsigned)(L.n_vt + n_split)), dim3(512), sm, st, a);
  e = hipGetLastError();
  if (e != hipSuccess || n_split == 0) return e;
  hipLaunchKernelGGL((k_items_tail<__bf16, 128, D>), dim3((128 * D) / 1024, (unsigned)n_split), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D, int NW>
static hipError_t items_launch(const Layout& L, char* ws, const void* E, const float* grad_loss, void* dE,
                               hipStream_t st) {
  if constexpr (narrow_owner(sizeof(T) == 2 ? 1 : 0, D)) {
    return items_launch16<D>(L, ws, E, grad_loss, dE, st);
  } else {
    using G = Geo<T, D, NW, true>;
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
    a.R_pad = L.R_pad;
    const size_t sm = two_pass<T, D>() && sizeof(T) == 4 ? G::kLdsBytes
                                                          : sweep_lds<T, D, NW, false, true, false, 0, 0>();
    // Two passes (see two_pass) run on the same grid and tail split. Measured: f32 D = 256 (the single pass
    // spills ~300 registers) 8.3 vs 21 ms.
    constexpr bool kTwoPass = two_pass<T, D>() && sizeof(T) == 4;
    constexpr auto kern = k_items<T, D, NW, kTwoPass ? 1 : 0>;
    constexpr auto kern2 = k_items<T, D, NW, kTwoPass ? 2 : 0>;
    int per_cu = 1;
    hipError_t e = kernel_setup<kern>(NW * 64, sm, per_cu);
    if (e != hipSuccess) return e;
    if (kTwoPass) {
      int c2 = 1;
      if ((e = kernel_setup<kern2>(NW * 64, sm, c2)) != hipSuccess) return e;
      if (c2 < per_cu) per_cu = c2;
    }
    // P workgroups run at once; tiles halved as halved_tiles says. The partial sums go to the forward sweep's
    // dH partial area, which is not in use during the backward dE sweep (it holds at least min(n_vt, 1024) tiles'
    // worth of rows x D floats; P <= 1024).
    const int64_t P = (int64_t)cu_count() * per_cu;
    const int64_t rem = L.n_vt % P;
    const int64_t n_split = halved_tiles(L.n_vt, P, rem, L.part_rows / (NW * 32) / 2);
    a.n_full = (int)(L.n_vt - n_split);
    a.tailpart = (float*)(ws + L.off_dhpart);
    if (n_split * 2 > (L.part_rows / (NW * 32))) return hipErrorInvalidValue;  // cannot happen: P <= 1024
    hipLaunchKernelGGL(kern, dim3((unsigned)(L.n_vt + n_split)), dim3(NW * 64), sm, st, a);
    e = hipGetLastError();
    if (e == hipSuccess && kTwoPass) {
      hipLaunchKernelGGL(kern2, dim3((unsigned)(L.n_vt + n_split)), dim3(NW * 64), sm, st, a);
      e = hipGetLastError();
    }
    if (e != hipSuccess || n_split == 0) return e;
    hipLaunchKernelGGL((k_items_tail<T, NW * 32, D>), dim3((NW * 32 * D) / 1024, (unsigned)n_split), dim3(256), 0, st,
                       a);
    return hipGetLastError();
  }
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
static hipError_t rows_any(const Layout& L, char* ws, const void* E, bool with_dh, bool met, bool pos_apply,
                           hipStream_t st) {
  if (met)
    return with_dh ? rows_launch<T, D, NW, true, true>(L, ws, E, st, pos_apply)
                   : rows_launch<T, D, NW, false, true>(L, ws, E, st, pos_apply);
  return with_dh ? rows_launch<T, D, NW, true, false>(L, ws, E, st, pos_apply)
                 : rows_launch<T, D, NW, false, false>(L, ws, E, st, pos_apply);
}

hipError_t launch_rows_sweep(const Layout& L, char* ws, const void* E, bool with_dh, bool met, bool pos_apply,
                             hipStream_t st) {
  CUTBCE_DISPATCH(L.dtype, rows_any, L, ws, E, with_dh, met, pos_apply, st);
}

template <typename T, int D, int NW>
static hipError_t topk_any(const Layout& L, char* ws, const void* E, int kt, hipStream_t st) {
  if (kt != kTopKMax) return hipErrorInvalidValue;
  return rows_launch<T, D, NW, false, false, kTopKMax>(L, ws, E, st);
}

hipError_t launch_topk_sweep(const Layout& L, char* ws, const void* E, int kt, hipStream_t st) {
  CUTBCE_DISPATCH(L.dtype, topk_any, L, ws, E, kt, st);
}

hipError_t launch_items_sweep(const Layout& L, char* ws, const void* E, const float* grad_loss, void* dE,
                              hipStream_t st) {
  CUTBCE_DISPATCH(L.dtype, items_launch, L, ws, E, grad_loss, dE, st);
}

}  // namespace cutbce
