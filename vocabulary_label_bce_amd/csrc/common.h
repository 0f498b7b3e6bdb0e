// Shared definitions of the gfx950 CutBCE library: element traits, MFMA wrappers, the re-laid-out operand
// formats, the workspace layout and the kernel launchers that api.hip calls.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cutbce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Tile geometry shared by the kernels.
constexpr int kWaveRows = 32;   // rows (or items) a wave owns in a sweep: one 32x32 MFMA tile edge
constexpr int kStep = 32;       // items (or rows) streamed per inner step: one 32x32 MFMA tile edge
constexpr int kPad = 256;       // R and V are padded to multiples of this inside the workspace
constexpr int kMaxSplits = 64;  // most vocabulary splits the forward sweep uses

// ---------------------------------------------------------------------------------------------------------
// Element traits. For a 32x32 output tile, lane l of a wave holds C/D register i (0..15) at
//   row  m = (i/4)*8 + (l/32)*4 + (i%4),  column n = l%32.
// bf16: v_mfma_f32_32x32x16_bf16 takes 8 consecutive k per lane: A[m=l%32][k=(l/32)*8+j], B[k=(l/32)*8+j][n=l%32].
// f32 : v_mfma_f32_32x32x2_f32 takes 1 k per lane: A[m=l%32][k=l/32], B[k=l/32][n=l%32].
// ---------------------------------------------------------------------------------------------------------
template <typename T> struct Elem;

template <> struct Elem<__bf16> {
  using Op = bf16x8;                 // one MFMA operand per lane
  static constexpr int kK = 16;      // k per MFMA
  static constexpr int kEPL = 8;     // elements per lane per operand
  static constexpr int kGroups = 2;  // MFMAs that consume the 16 accumulator registers of one 32x32 tile
  __device__ static inline f32x16 mma(Op a, Op b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Elem<float> {
  using Op = float;
  static constexpr int kK = 2;
  static constexpr int kEPL = 1;
  static constexpr int kGroups = 16;
  __device__ static inline f32x16 mma(Op a, Op b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Position (0..31) inside a 32-element block of the row/column that accumulator register i of a lane in
// half h (= l/32) belongs to. Used to re-lay out the streamed operand of the second GEMM so that the
// accumulator tile of the first GEMM can be fed back as an MFMA operand without any shuffle: the k order of
// the second GEMM is permuted to match (a reduction is invariant under a common permutation of k).
__host__ __device__ constexpr inline int acc_pos(int i, int h) { return (i / 4) * 8 + h * 4 + (i % 4); }

// "Slot-packed" layout of a [32 x D] block X (32 rows/items, D features) for the second GEMM's B operand:
// for d-block db (32 features) and MFMA group g, lane l reads kEPL consecutive elements
//   X[acc_pos(g*kEPL + j, l/32)][db*32 + l%32],  j = 0..kEPL-1
// stored contiguously, lane-major. Offset (in elements) of that run inside the block:
template <typename T>
__host__ __device__ constexpr inline int64_t slot_off(int D, int db, int g, int lane) {
  return ((int64_t)(db * Elem<T>::kGroups + g) * 64 + lane) * Elem<T>::kEPL;
}

// ---------------------------------------------------------------------------------------------------------
// Workspace layout (computed on the host, passed by value to kernels that need pointers into it).
// ---------------------------------------------------------------------------------------------------------
struct Ctl {           // device control block
  int32_t n_valid;     // R_v, the number of valid rows
  int32_t splits;      // vocabulary splits chosen by the forward sweep
  int32_t bad_ids;     // ids skipped by the bucketing kernels (out of range)
  int32_t pad0;
  double scale;        // s = 1 / (W * V), W = summed weight of the valid rows (R_v without weights); 0 when W == 0
  uint32_t hnorm_max;  // bits of max_r ||H[r]|| over the valid rows (a non-negative float), set by the H preparation
  uint32_t hw_absmax;  // bits of max |w_r H[r][d]| over the valid rows (the f16 gradient operand's scale)
  uint32_t enorm_max;  // bits of max_v ||E[v]|| (from the E preparation's statistics, f16-Evp shapes)
  uint32_t e_absmax;   // bits of max |E[v][d]| (same)
  int32_t evp_shift;   // the power of two the f16 Evp holds E scaled by; kept from call to call (not reset)
  int32_t evp_fix;     // 1 when this call's E needs another scale than the previous call's: Evp is rewritten
};

// Shapes whose dE sweep runs its gradient GEMM in f16 (every bf16 input): the slot-packed rows Hrp are stored as
// f16, scaled by 2^hrp_shift(hw_absmax), and the G tiles c = sigma(z) - 1/2 - y are f16 (c - 1 at a positive
// keeps 10 fraction bits instead of bf16's 7).
__host__ __device__ constexpr inline bool hrp_is_f16(int dtype, int D) { return dtype == 1 && D > 0; }

// Shapes whose sweeps run on the 16-owner engine (bf16, D = 256 and 512): a wave owns 16 rows or items and the
// MFMAs are 16x16x32 tiles (lane l supplies A[m = l%16][k = 8(l/16) + j] and B[k = 8(l/16) + j][n = l%16], j < 8,
// and holds D[m = 4(l/16) + i][n = l%16], i < 4). Its slot-packed copies (Evp, Hrp) of a 32-row block X use:
// for 16-wide d-block db and lane l, the 8 elements X[sp16_row(l, j)][16 db + l % 16] (j = 0..7) stored together.
__host__ __device__ constexpr inline bool narrow_owner(int dtype, int D) { return dtype == 1 && D >= 256; }

// Shapes whose forward sweep runs its gradient GEMM in f16 (bf16 input on the 32-owner engines, D <= 128): the
// slot-packed E copy Evp is stored as f16 scaled by 2^evp_shift, the G tiles are f16, and the dH partials are
// multiplied by 2^-evp_shift when written. The E preparation writes Evp with the previous call's shift and takes
// max ||E[v]|| and max |E| on the way; the shift stands if it puts max |E| in [2^13, 2^15), else a second pass
// rewrites Evp with the shift that puts it in [2^14, 2^15). The norm bound also lets the forward sweep take its
// polynomial epilogue.
__host__ __device__ constexpr inline bool evp_is_f16(int dtype, int D) { return dtype == 1 && D <= 128; }
__host__ __device__ constexpr inline int sp16_row(int lane, int j) { return 16 * (j / 4) + 4 * (lane / 16) + (j % 4); }
__host__ __device__ constexpr inline int64_t sp16_off(int db, int lane) { return ((int64_t)db * 64 + lane) * 8; }

// Power of two that brings the largest |w_r H[r][d]| into [2^14, 2^15) (0 when every value is 0), so that the f16
// copy keeps 11 significant bits for every value within 2^29 of the largest.
__device__ inline int hrp_shift(uint32_t absmax_bits) {
  const float m = __uint_as_float(absmax_bits);
  if (!(m > 0.f)) return 0;
  int e = 0;
  (void)frexpf(m, &e);  // m = f * 2^e, f in [0.5, 1)
  const int k = 15 - e;
  return k < -120 ? -120 : (k > 120 ? 120 : k);
}

// The shift an f16 Evp was written with (clamped, so that a workspace that never held one gives a finite scale).
__device__ inline int evp_shift_of(const Ctl* ctl) {
  const int k = ctl->evp_shift;
  return k < -120 ? -120 : (k > 120 ? 120 : k);
}

struct Layout {
  int64_t R, V, nnz;
  int D, dtype, esz;
  int64_t R_pad, V_pad;
  int64_t n_rt;       // row tiles of the forward sweep (R_pad / rows_per_wg)
  int64_t n_vt;       // item tiles of the backward sweep (V_pad / items_per_wg)
  int64_t n_rs, n_vs; // 32-row / 32-item steps
  int rows_per_wg, items_per_wg;
  int64_t n_eblk;     // blocks of the E preparation kernel
  int64_t nb_r, nb_i; // bucket counts (forward: row tile x item step; backward: item tile x row step)
  size_t off_ctl, off_row_of, off_compact_of, off_rptr, off_wc, off_Hc, off_Hrp, off_sumH, off_sumH_part;
  size_t off_sumE, off_sumE_part, off_sum2, off_Evp, off_dhpart, off_rowpart, off_metpart, off_rowloss, off_dhtmp;
  size_t off_estat;  // per-block maxima of the E statistics (two floats per E preparation block)
  size_t off_rowform;  // per compacted row: 1 if the forward's waves took the polynomial epilogue (bf16, D <= 128)
  size_t off_bptr_r, off_bfill_r, off_pairs_r, off_bptr_i, off_bfill_i, off_pairs_i, off_scan, off_cpart;
  size_t scan_elems;
  int64_t part_rows;  // rows of the forward sweep's unit-major partial buffers
  size_t total;
};

#ifndef CUTBCE_GATHER_POSITIVES
#define CUTBCE_GATHER_POSITIVES 1
#endif
// Where the forward takes its positives (the sparse target correction of the loss and of dH): gathered per row
// by the finishing kernel (1), or bucketed and folded into the sweep's tiles (0). With Cut Metrics the buckets
// are built either way (the counts need each positive's logit), and with 1 the sweep only counts them.
constexpr bool kGatherPositives = CUTBCE_GATHER_POSITIVES != 0;

constexpr int kEBlkItems = 256;   // items per block of the E preparation kernel (column-sum granularity)
constexpr int kScanBlock = 8192;  // elements per block of the multi-block scan
constexpr int kSumMaxGroups = 64;  // part groups of the two-pass column sums (group sums: kSumMaxGroups x D doubles)

// Waves per workgroup of the 32-owner sweeps for a (dtype, D); a workgroup's row tile (and, except for the
// 16-owner dE sweep, item tile) is 32 of these. bf16 D = 512: only the scoring sweep runs on it, with the row tiles
// of the 16-owner forward (64 rows).
__host__ __device__ constexpr inline int sweep_waves(int dtype, int D) {
  return (dtype == 1) ? (D <= 128 ? 8 : (D == 256 ? 4 : 2)) : (D <= 64 ? 8 : 4);
}
// Waves per workgroup of the 16-owner forward (bf16, D >= 256): two per SIMD at D = 256; one at D = 512, where
// the owner operand and the dH accumulators take 192 registers and two waves would spill.
__host__ __device__ constexpr inline int rows16_waves(int D) { return D == 512 ? 4 : 8; }
// Item tile of the dE sweep: 8 waves x 16 items on the 16-owner engine, else 32 per wave.
__host__ __device__ constexpr inline int items_tile(int dtype, int D) {
  return narrow_owner(dtype, D) ? 128 : sweep_waves(dtype, D) * 32;
}

// ---------------------------------------------------------------------------------------------------------
// Launchers (each returns the hipError_t of its launches).
// ---------------------------------------------------------------------------------------------------------
hipError_t launch_compact(const Layout& L, char* ws, const uint8_t* mask, const float* weight,
                          const int32_t* row_offsets, hipStream_t st);
hipError_t launch_prep_h(const Layout& L, char* ws, const void* H, bool want_hrp, hipStream_t st);
// The dE sweep's slot-packed rows Hrp from a workspace whose row compaction and H preparation are done (bf16: the
// f16 copy from Hc and the row statistics; f32: the H preparation again, with Hrp).
hipError_t launch_prep_hrp(const Layout& L, char* ws, const void* H, hipStream_t st);
hipError_t launch_prep_e(const Layout& L, char* ws, const void* E, bool want_evp, hipStream_t st);
hipError_t launch_buckets(const Layout& L, char* ws, const int32_t* item_ids, bool rows_side, hipStream_t st);
// pos_apply: the positives of the buckets enter the tiles (c - 1 and the sum of their logits); false: with Cut
// Metrics they are only counted (the finish gathers their terms), without it the buckets are empty anyway.
hipError_t launch_rows_sweep(const Layout& L, char* ws, const void* E, bool with_dh, bool met, bool pos_apply,
                             hipStream_t st);
// E != nullptr: the forward sweep ran without positives and the finish gathers them (sum of the positives'
// logits for the loss, minus the sum of their E rows for dH); E == nullptr: the sweep's partials include them.
hipError_t launch_rows_finish(const Layout& L, char* ws, const void* H, const uint8_t* mask, float* loss,
                              float* row_loss, float* dh_out, bool with_dh, int32_t* metrics, const void* E,
                              const int32_t* item_ids, hipStream_t st);
// Bucket pointers of the forward sweep set to zero (every bucket empty, the sweep sees no positives) for the
// sweeps that read them; the bf16 forward sweeps without Cut Metrics read none, and nothing is launched for them.
hipError_t launch_no_row_buckets(const Layout& L, char* ws, hipStream_t st);
hipError_t launch_items_sweep(const Layout& L, char* ws, const void* E, const float* grad_loss, void* dE,
                              hipStream_t st);
// full-vocabulary scoring: per-split top-kt lists (kt = kTopKMax entries kept) in the dH partial area
constexpr int kTopKMax = 8;  // largest k of the scoring path (the paper evaluates Hit@8)
hipError_t launch_topk_sweep(const Layout& L, char* ws, const void* E, int kt, hipStream_t st);
hipError_t launch_topk_finish(const Layout& L, char* ws, const uint8_t* mask, const int32_t* item_ids, int kt, int k,
                              float* vals, int32_t* ids, int32_t* hits, hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t st);
hipError_t launch_scale_dh(const Layout& L, const float* src, const float* grad_loss, void* dH, hipStream_t st);
hipError_t launch_targets_to_csr(int64_t R, int L, const int32_t* targets, int32_t pad, int32_t* row_offsets,
                                 int32_t* item_ids, hipStream_t st);
hipError_t launch_validate(int64_t R, int64_t V, int64_t nnz, const int32_t* row_offsets,
                           const int32_t* item_ids, int32_t* bad, hipStream_t st);

}  // namespace cutbce
