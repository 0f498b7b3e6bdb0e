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
// The forward sweep also serves full-vocabulary scoring (top-k per row, Section I-E's evaluation) with a
// running top list per lane in place of the loss epilogue, and can count the Cut Metrics of Section III-D.
#include <atomic>

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

// c_i = 1/w_i - 1/2 for 16 factors w_i >= 1 with pair products w2 and quad products w4 (each below 2^126):
// one reciprocal per quad, then down the product tree (batch inversion): 1/(w0 w1) = w2 w3 / (w0 w1 w2 w3),
// 1/w0 = w1 / (w0 w1), ...; each 1/w_i picks up two extra roundings.
__device__ inline void inv_minus_half(const float* w, const float* w2, const float* w4, float* c) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
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
//    bf16 D = 512 forward, whose one wave per SIMD has 512 registers: its 128 registers of A operands spill
//    about 35 others, and still save 17% against reading each operand next to its MFMA, 4.56 vs 5.51 ms at
//    4,096 rows x 262,144 items): iteration i runs the logit GEMM of step i on A operands read from LDS
//    during iteration i-1, reads those of step i+1, and evaluates the epilogue of step i;
//  - otherwise the logit GEMM of step i+1 runs in iteration i with its A operands read next to each MFMA, two
//    logit tiles alternating, and the epilogue of step i uses the tile formed in iteration i-1.
// Ring loads, their slots and the barrier every kK iterations follow Geo; bucket pointers come 64 steps at a
// time (bkt_*), their refill riding on a barrier iteration.
// ---------------------------------------------------------------------------------------------------------
// DB0, NDBE: the gradient GEMM covers the d-blocks [DB0, DB0 + NDBE) of the 32-wide blocks of D (acc holds
// NDBE tiles); LOSS = false skips the loss sums of the forward epilogue (a second pass over the other d-blocks).
template <typename T, int D, int NW, bool FWD, bool GRAD, bool MET = false, int KT = 0, int DB0 = 0,
          int NDBE = D / 32, bool LOSS = true>
struct Engine {
  using EL = Elem<T>;
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

    GPack<T> g;  // G tile whose gradient GEMM is pending
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
  __device__ inline void step_lds(int i, const Op* own, const f32x16& zc, f32x16& zn, GPack<T>& g, f32x16* acc,
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

  __device__ inline void grad(int j, const GPack<T>& g, f32x16* acc) const {
    grad_slot(j % (G::kNB ? G::kNB : 1), g, acc);
  }
  __device__ inline void grad_slot(int slot, const GPack<T>& g, f32x16* acc) const {
    const char* b = lds + (G::kNA + slot) * G::kStepBytes;
#pragma unroll
    for (int db = 0; db < NDBE; ++db)
#pragma unroll
      for (int q = 0; q < EL::kGroups; ++q)
        acc[db] = EL::mma(g.op(q), lds_b<T, D>(b, DB0 + db, q, lane), acc[db]);
  }

  // Epilogue of step j (called for j = 0, 1, ... in order): positives of the step (bucket [pb, pe)),
  // loss sums (FWD), the G tile (GRAD) and, with MET, the Cut Metrics counts of the lane: met[0] logits
  // predicted positive (z > 0), met[1] positives predicted positive, met[2] positives.
  __device__ inline void epilogue(int j, int pb, int pe, const f32x16& z, GPack<T>& g, float& e_acc, float& posz,
                                  int* met, TopK<KT ? KT : 1>* tk) {
    if constexpr (KT > 0) {
      // scoring: keep the lane's best items (real items only; the last step may hold padding). Only the values
      // above the lane's current k-th best are inserted, one at a time, picked by a select chain (no dynamic
      // register indexing). Items past the vocabulary exist only in its last step: the lane's bound (32-bit,
      // V < 2^31) is all-pass elsewhere.
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
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (pm & (1u << q)) {
            if (FWD) posz += z[q];
            c[q] -= 1.f;
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
  float* topv;     // [units][RW][KT]: per-split top-KT logits (scoring)
  int32_t* topi;   // [units][RW][KT]: their item ids
};

// ---------------------------------------------------------------------------------------------------------
// Forward sweep. Persistent: gridDim.x workgroups (as many as can be resident, a multiple of 8); units (split s,
// row tile t) are assigned in contiguous per-XCD ranges so that the workgroups sharing an L2 stream the same
// part of E. With KT > 0 it scores instead: per-lane top-KT lists, merged per row and written per unit.
// ---------------------------------------------------------------------------------------------------------
// DHPART 0: one pass (loss, dH and optional Cut Metrics); 1 / 2: the first / second of two passes, each
// accumulating half of dH's d-blocks (half the accumulator registers, for D = 512); the loss and the Cut
// Metrics come from pass 1.
template <typename T, int D, int NW, bool WITH_DH, bool MET, int KT, int DHPART = 0>
__global__ void __launch_bounds__(NW * 64) k_rows(RowsArgs a) {
  using EL = Elem<T>;
  constexpr int NDB = D / 32, NDBE = DHPART ? NDB / 2 : NDB, DB0 = DHPART == 2 ? NDB / 2 : 0;
  using EN = Engine<T, D, NW, true, WITH_DH, MET, KT, DB0, NDBE, DHPART != 2>;
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

  EN en;
  en.setup(lds, wave, lane);
  en.X = (const T*)a.E;
  en.Xsp = (const T*)a.Evp;
  en.nX = a.V;
  en.bptr = a.bptr;
  en.pairs = a.pairs;

  for (int idx = slot; idx < cnt; idx += P / 8) {
    const int u = start + idx;
    const int s = u / Tt, t = u % Tt;
    en.j0 = (int)(((int64_t)s * n_steps) / S);
    en.j1 = (int)(((int64_t)(s + 1) * n_steps) / S);
    const int r_base = t * RW + wave * 32;
    en.bbase = (int64_t)t * a.n_vs;
    en.own0 = r_base;

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
    if (MET) {
#pragma unroll
      for (int q = 0; q < 3; ++q) met[q] += __shfl_xor(met[q], 32, 64);
      if (lane < 32) a.metpart[urow + lane] = make_int4(met[0], met[1], met[2], 0);
    }
    if (WITH_DH) {
#pragma unroll
      for (int db = 0; db < NDBE; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          a.dhpart[(urow + acc_pos(i, lane / 32)) * D + (DB0 + db) * 32 + lane % 32] = acc[db][i];
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
  int n_full;        // item tiles swept whole; the tiles after them are swept in two row halves
  float* tailpart;   // [split tile][half][IW][D] fp32 partial sums of the halved tiles
};

// ---------------------------------------------------------------------------------------------------------
// Backward dE sweep: workgroup = item tile (32 items per wave), sweeping all valid rows.
// ---------------------------------------------------------------------------------------------------------
// DEPART 0: one pass; 1 / 2: the first / second of two passes, each accumulating and writing half of dE's
// d-blocks (half the accumulator registers, for D = 512).
template <typename T, int D, int NW, int DEPART = 0>
__global__ void __launch_bounds__(NW * 64) k_items(ItemsArgs a) {
  using EL = Elem<T>;
  constexpr int NDB = D / 32, NDBE = DEPART ? NDB / 2 : NDB, DB0 = DEPART == 2 ? NDB / 2 : 0;
  using EN = Engine<T, D, NW, false, true, false, 0, DB0, NDBE>;
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

  const int n_valid = a.ctl->n_valid;
  const int n_st = (n_valid + 31) / 32;
  if (n_st > 0) {
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

  // dE[v][d] = s * g * (acc + 1/2 sum_r H[r][d])
  const double sc = a.ctl->scale * (double)a.grad_loss[0];
  const float scf = (float)sc;
  T* __restrict__ dE = (T*)a.dE;
#pragma unroll
  for (int db = 0; db < NDBE; ++db) {
    const int d = (DB0 + db) * 32 + lane % 32;
    const float half = (float)(0.5 * a.sumH[d]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t v = v_own0 + acc_pos(i, lane / 32);
      if (v < a.V) dE[v * D + d] = (T)(scf * (acc[db][i] + half));
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
  const float q[4] = {p0.x + p1.x, p0.y + p1.y, p0.z + p1.z, p0.w + p1.w};
  T* __restrict__ out = (T*)a.dE + v * D + d;
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = (T)(scf * (q[k] + (float)(0.5 * a.sumH[d + k])));
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
// when they fill the 256 registers of a wave, the sweep can run as two passes over half of the gradient's
// d-blocks each (bf16 D = 512, f32 D = 256), recomputing the logits instead of spilling. Measured, forward:
// bf16 D = 512 4.95 -> 2.47 ms, f32 D = 256 26.4 -> 17.2 ms (4,096 rows, 131,072 items).
template <typename T, int D>
constexpr bool two_pass() {
  return (D / 32) * 16 + (D / Elem<T>::kK) * (int)(sizeof(typename Elem<T>::Op) / 4) >= 256;
}

// Forward-sweep grid: persistent, as many workgroups as can be resident at once (per_cu per CU), a multiple of
// 8 (one range per XCD). The kernel derives its vocabulary splits from the grid size.
static int persistent_grid(int per_cu) {
  const int P = (cu_count() * per_cu / 8) * 8;
  return P > 0 ? P : 8;
}

template <typename T, int D, int NW, bool WITH_DH, bool MET, int KT = 0>
static hipError_t rows_launch(const Layout& L, char* ws, const void* E, hipStream_t st) {
  using G = Geo<T, D, NW, WITH_DH>;
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
  a.metpart = (int4*)(ws + L.off_metpart);
  // scoring partials reuse the dH partial area: KT * 8 bytes per row <= D * 4 bytes
  static_assert(KT * 8 <= D * 4, "top-k partials fit in the dH partial area");
  a.topv = (float*)(ws + L.off_dhpart);
  a.topi = (int32_t*)(ws + L.off_dhpart) + (size_t)L.part_rows * (KT ? KT : 1);
  const size_t sm = G::kLdsBytes;
  // Both passes run on the same grid, hence the same vocabulary splits and partial-sum layout.
  constexpr bool kTwoPass = WITH_DH && KT == 0 && two_pass<T, D>();
  if constexpr (kTwoPass) {
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
    int per_cu = 1;
    hipError_t e = kernel_setup<kern>(NW * 64, sm, per_cu);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(persistent_grid(per_cu)), dim3(NW * 64), sm, st, a);
    return hipGetLastError();
  }
}

template <typename T, int D, int NW>
static hipError_t items_launch(const Layout& L, char* ws, const void* E, const float* grad_loss, void* dE,
                               hipStream_t st) {
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
  const size_t sm = G::kLdsBytes;
  // Two passes (see two_pass) run on the same grid and tail split. Measured: f32 D = 256 (the single pass
  // spills ~300 registers) 8.3 vs 21 ms; bf16 D = 512 (~100 spilled) is faster in one pass, 1.87 vs 2.03 ms.
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
  // P workgroups run at once; when the last round would be at most half full, its tiles are halved. The
  // partial sums go to the forward sweep's dH partial area, which is not in use during the backward dE sweep
  // (it holds at least 1024 tiles' worth of rows x D floats; P <= 1024).
  const int64_t P = (int64_t)cu_count() * per_cu;
  const int64_t rem = L.n_vt % P;
  const int64_t n_split = (L.n_vt > P && rem > 0 && 2 * rem <= P) ? rem : 0;
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
static hipError_t rows_any(const Layout& L, char* ws, const void* E, bool with_dh, bool met, hipStream_t st) {
  if (met)
    return with_dh ? rows_launch<T, D, NW, true, true>(L, ws, E, st) : rows_launch<T, D, NW, false, true>(L, ws, E, st);
  return with_dh ? rows_launch<T, D, NW, true, false>(L, ws, E, st) : rows_launch<T, D, NW, false, false>(L, ws, E, st);
}

hipError_t launch_rows_sweep(const Layout& L, char* ws, const void* E, bool with_dh, bool met, hipStream_t st) {
  CUTBCE_DISPATCH(L.dtype, rows_any, L, ws, E, with_dh, met, st);
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
