// Shared definitions of the gfx950 CutBCE library: element traits, MFMA wrappers, the re-laid-out operand
// formats, the workspace layout and the kernel launchers that api.hip calls.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cutbce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
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
};

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
  size_t off_sumE, off_sumE_part, off_Evp, off_dhpart, off_rowpart, off_metpart, off_rowloss, off_dhtmp;
  size_t off_bptr_r, off_bfill_r, off_pairs_r, off_bptr_i, off_bfill_i, off_pairs_i, off_scan;
  size_t scan_elems;
  int64_t part_rows;  // rows of the forward sweep's unit-major partial buffers
  size_t total;
};

constexpr int kEBlkItems = 256;   // items per block of the E preparation kernel (column-sum granularity)
constexpr int kScanBlock = 8192;  // elements per block of the multi-block scan

// Launch configuration of the two sweeps for a (dtype, D): waves per workgroup.
__host__ __device__ constexpr inline int sweep_waves(int dtype, int D) {
  return (dtype == 1) ? (D <= 128 ? 8 : 4) : (D <= 64 ? 8 : 4);
}

// ---------------------------------------------------------------------------------------------------------
// Launchers (each returns the hipError_t of its launches).
// ---------------------------------------------------------------------------------------------------------
hipError_t launch_compact(const Layout& L, char* ws, const uint8_t* mask, const float* weight,
                          const int32_t* row_offsets, hipStream_t st);
hipError_t launch_prep_h(const Layout& L, char* ws, const void* H, bool want_hrp, hipStream_t st);
hipError_t launch_prep_e(const Layout& L, char* ws, const void* E, bool want_evp, hipStream_t st);
hipError_t launch_buckets(const Layout& L, char* ws, const int32_t* item_ids, bool rows_side, hipStream_t st);
hipError_t launch_rows_sweep(const Layout& L, char* ws, const void* E, bool with_dh, bool met, hipStream_t st);
hipError_t launch_rows_finish(const Layout& L, char* ws, const void* H, const uint8_t* mask, float* loss,
                              float* row_loss, float* dh_out, bool with_dh, int32_t* metrics, hipStream_t st);
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
